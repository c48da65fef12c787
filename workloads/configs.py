"""Workload shapes for the verify path (synthetic stand-ins for the pages' serving loads).

Every workload is synthetic: the pages measure on gsm8k / arena-hard / poetry traffic and
on Qwen3 / DeepSeek serving loads, none of which is available here.  The shapes below
follow those loads (batch, block length, GQA geometry, paged bf16 KV, vocabulary), the
value distributions are seeded draws described in ``generate.py``.

This module holds sizes and cost tables only -- none of the method's arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass, field

# Step-cost line of the SGLang article ("Background" figure caption): T(M) = 20 ms +
# 0.19 ms per verify token; used as bias = 20, alpha(bs) = 0, theta(M) = 0.19 M.
BIAS_MS = 20.0
THETA_MS_PER_TOKEN = 0.19

# High-concurrency workload: theta per token chosen so that the seeded draw's mean window
# is 3 (windows "shrink to 2-4").  Found by bisection with the oracle's scheduler by
# tests/golden/make_theta_high_concurrency.py; test_workloads checks it is current.
THETA_HIGH_CONCURRENCY = 0.06617


@dataclass(frozen=True)
class ConfClass:
    """One traffic class: confidences c ~ Beta(a, b).  sigma: the draft-logit noise std at
    the class's mean confidence (the synthetic acceptance traces of the STS benchmark use it;
    the workloads' draft rows take each draft's own sigma from its drawn confidence)."""

    a: float
    b: float
    sigma: float


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    gamma: int                      # block length, anchor included
    classes: tuple                  # ConfClass per class; requests assigned round-robin
    conf_from_head: bool            # True: hidden states + linear head; False: c given
    head_H: int                     # hidden size of the confidence head (head mode)
    Hq: int
    Hkv: int
    D: int
    kv_dtype: str                   # "bf16" | "f32"
    page: int
    ctx_lo: int
    ctx_hi: int                     # contexts ~ U[ctx_lo, ctx_hi] (inclusive)
    V: int
    logit_dtype: str                # "bf16" | "f32"
    pack_hidden: int                # row width of the packed hidden buffer (stage 2)
    tiers: tuple
    theta_ms_per_token: float
    seed: int
    bias_ms: float = BIAS_MS
    description: str = ""
    target_logit_std: float = 2.0
    extra: dict = field(default_factory=dict)

    @property
    def G1(self):
        return self.gamma - 1

    @property
    def max_pages(self):
        return -(-(self.ctx_hi + self.gamma) // self.page)


def _mult(step, top):
    return tuple(range(step, top + 1, step))


WORKLOADS = {
    "tiny": Workload(
        name="tiny", B=4, gamma=6, classes=(ConfClass(8, 2, 0.5),), conf_from_head=False,
        head_H=0, Hq=4, Hkv=2, D=64, kv_dtype="f32", page=16, ctx_lo=64, ctx_hi=256, V=1024,
        logit_dtype="f32", pack_hidden=256, tiers=(4, 8, 12, 16, 24),
        theta_ms_per_token=THETA_MS_PER_TOKEN, seed=1000,
        description="Tiny: B=4, gamma=6, GQA 4/2 D=64 fp32 KV page 16, ctx U[64,256], V=1024"),
    "qwen3-4b": Workload(
        name="qwen3-4b", B=16, gamma=6, classes=(ConfClass(8, 2, 0.5),), conf_from_head=True,
        head_H=2560, Hq=32, Hkv=8, D=128, kv_dtype="bf16", page=64, ctx_lo=1024, ctx_hi=4096,
        V=151936, logit_dtype="bf16", pack_hidden=2560, tiers=_mult(8, 128),
        theta_ms_per_token=THETA_MS_PER_TOKEN, seed=1001,
        description="Qwen3-4B-like verify shapes: B=16, gamma=6, GQA 32/8 D=128 bf16 page 64, "
                    "ctx U[1K,4K], confidence head H=2560, V=151936 bf16"),
    "mixed-b64": Workload(
        name="mixed-b64", B=64, gamma=8,
        classes=(ConfClass(19, 1, 0.125), ConfClass(9, 1, 0.25), ConfClass(4, 1, 0.5)),
        conf_from_head=False, head_H=0, Hq=32, Hkv=8, D=128, kv_dtype="bf16", page=64,
        ctx_lo=512, ctx_hi=8192, V=151936, logit_dtype="bf16", pack_hidden=4096,
        tiers=_mult(8, 512), theta_ms_per_token=THETA_MS_PER_TOKEN, seed=1002,
        description="Mixed traffic B=64: 3 classes Beta(19,1)/Beta(9,1)/Beta(4,1), gamma=8, "
                    "GQA 32/8 D=128 bf16 page 64, ctx U[512,8K], V=151936 bf16"),
    "high-conc-b256": Workload(
        name="high-conc-b256", B=256, gamma=16, classes=(ConfClass(6, 1.5, 0.5),),
        conf_from_head=False, head_H=0, Hq=32, Hkv=8, D=128, kv_dtype="bf16", page=64,
        ctx_lo=2048, ctx_hi=2048, V=151936, logit_dtype="bf16", pack_hidden=4096,
        tiers=_mult(8, 4096), theta_ms_per_token=THETA_HIGH_CONCURRENCY, seed=1003,
        description="High concurrency B=256: gamma=16, Beta(6,1.5), GQA 32/8 D=128 bf16 page 64, "
                    "ctx 2048, V=151936 bf16, theta tuned for windows of 2-4"),
    "long-b32": Workload(
        name="long-b32", B=32, gamma=8, classes=(ConfClass(9, 1, 0.25),), conf_from_head=False,
        head_H=0, Hq=64, Hkv=8, D=128, kv_dtype="bf16", page=64, ctx_lo=16384, ctx_hi=32768,
        V=151936, logit_dtype="bf16", pack_hidden=8192, tiers=_mult(8, 256),
        theta_ms_per_token=THETA_MS_PER_TOKEN, seed=1004,
        description="Long context B=32: gamma=8, Beta(9,1), GQA 64/8 D=128 bf16 page 64, "
                    "ctx U[16K,32K], V=151936 bf16"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
