"""Seeded synthetic inputs for the verify path.

The ONLY code shared by the HIP path's harness and the oracle's tests.  It draws inputs
and lays them out; it contains none of the method's arithmetic (no softmax, no survival
product, no scheduling, no acceptance).

Recipe (NumPy PCG64; every (request, array) pair has its own SeedSequence spawn key, so
any request can be regenerated alone and arrays are independent of each other):

* contexts L_b ~ U[ctx_lo, ctx_hi] (integers, inclusive); classes round-robin over b.
* confidences c[b, k] ~ Beta(a, b) of the request's class (float32), or, for the
  confidence-head workload, hidden states built so that the head's logit is
  z = log(c / (1 - c)) for c ~ Beta(a, b): head weights w ~ N(0, 1/H) (float32),
  h = g + ((z - w.g) / (w.w)) w with g ~ N(0, I), rounded to bf16 (the head output is
  recomputed from the rounded h by whoever consumes it).
* q, k_new, v_new (all gamma block positions) and the cached context K/V: N(0, 1),
  rounded to the KV dtype.
* target logits: N(0, std^2) per row (gamma rows per request, std = 2); draft row k =
  target row k-1 + N(0, sigma_k^2); both rounded to the logit dtype.  sigma_k follows the
  request's drawn confidence c_k for draft k, so that the draft is accepted with probability
  c_k: with n ~ N(0, sigma^2) added to every logit, p_d / p_t = exp(n - sigma^2 / 2) under
  p_t, whose expected overlap sum_v min(p_t, p_d) is 2 Phi(-sigma / 2) for a large
  vocabulary; sigma_k = -2 Phi^-1(c_k / 2) (0.125, 0.25, 0.5 at c = 0.95, 0.9, 0.8).
* draft tokens: drawn from softmax(draft row) with the Gumbel-max trick in float64
  (argmax of logits + Gumbel noise), i.e. a sample of the drafter, not part of the path.
* u_accept[b, k], u_resample[b]: U[0, 1) float32.
* packed-buffer source rows (stage 2): N(0, 1) bf16, [gamma, pack_hidden] per request.
* page table: request b owns ceil((L_b + gamma) / page) pages; the physical page numbers
  are a seeded permutation of all pages (a fragmented pool).
* calibration traces (``calibration_trace``): per sample and draft position a true
  conditional acceptance probability q ~ Beta(a, b) (float64); the head logit is
  z = T_k * log(q / (1 - q)) + noise * N(0, 1), rounded to float32 (T_k > 1: an
  over-confident head); draft k is accepted iff U[0, 1) < q, and the accept length is the
  number of leading accepted drafts; the observed length is gamma - 1 (full-block runs) or,
  censored, U{0 .. gamma-1} (compact runs, which verify only the window).
* Markov-head inputs (``markov_inputs``): base logits U [B, gamma-1, V] ~ N(0, 2^2) in the
  logit dtype; anchors uniform over the vocabulary; uniforms U[0, 1) float32; the rank-r
  factors as int8 uniform on [-127, 127] ([V, r] each: embedding rows and vocabulary rows)
  with float32 scales 4.2e-3 * U[0.5, 1.5] per row (a bias of standard deviation about
  1.5 at r = 256).
"""

from __future__ import annotations

from statistics import NormalDist

import numpy as np
import torch

from .configs import Workload

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def draft_sigma(c: np.ndarray) -> np.ndarray:
    """Draft-logit noise std (float32) at which a draft is accepted with probability c:
    sigma = -2 Phi^-1(c / 2), clamped to c in [1e-6, 1 - 1e-6]."""
    nd = NormalDist()
    cc = np.clip(np.asarray(c, np.float64), 1e-6, 1.0 - 1e-6)
    return np.array([-2.0 * nd.inv_cdf(x / 2.0) for x in cc], np.float32)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array -> torch CPU tensor of the dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_TORCH[dtype])


class Inputs:
    """Lazily generated inputs of one workload."""

    # grandchild index per array kind
    _QKV, _CTX, _LOGITS, _GUMBEL, _UNIF, _PACK, _CONF = range(7)

    def __init__(self, wl: Workload, seed: int | None = None, B: int | None = None):
        self.wl = wl
        self.seed = wl.seed if seed is None else seed
        self.B = wl.B if B is None else B
        # stateless derivation: spawn key (0,) is the batch-level stream, (1, b, kind) the
        # stream of array `kind` of request b
        g = np.random.default_rng(np.random.SeedSequence(self.seed, spawn_key=(0,)))
        B, wl = self.B, self.wl
        self.context_lens = g.integers(wl.ctx_lo, wl.ctx_hi + 1, size=B).astype(np.int32)
        self.classes = (np.arange(B) % len(wl.classes)).astype(np.int32)
        self.pages_per_req = -(-(self.context_lens.astype(np.int64) + wl.gamma) // wl.page)
        self.num_pages = int(self.pages_per_req.sum())
        self.max_pages = int(self.pages_per_req.max())
        perm = g.permutation(self.num_pages).astype(np.int32)
        self.block_table = np.zeros((B, self.max_pages), np.int32)
        k = 0
        for b in range(B):
            n = int(self.pages_per_req[b])
            self.block_table[b, :n] = perm[k:k + n]
            k += n
        if wl.conf_from_head:
            self.head_w = (g.standard_normal(wl.head_H) / np.sqrt(wl.head_H)).astype(np.float32)
            self.head_b = np.float32(0.0)
        else:
            self.head_w = None
            self.head_b = np.float32(0.0)
        self._cache = {}

    # ------------------------------------------------------------------ helpers
    def _rng(self, b: int, kind: int) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence(self.seed, spawn_key=(1, b, kind)))

    def cls(self, b):
        return self.wl.classes[int(self.classes[b])]

    # ------------------------------------------------------------------ stage 1 inputs
    def conf64(self, b: int) -> np.ndarray:
        """Request b's drawn confidences [gamma-1] (float64): the Beta draw behind both the
        given confidences and the head's hidden states."""
        c = self.cls(b)
        return self._rng(b, self._CONF).beta(c.a, c.b, size=self.wl.G1)

    def conf(self) -> np.ndarray:
        """[B, gamma-1] float32 confidences (beta workloads)."""
        if "conf" not in self._cache:
            out = np.empty((self.B, self.wl.G1), np.float32)
            for b in range(self.B):
                out[b] = self.conf64(b)
            self._cache["conf"] = out
        return self._cache["conf"]

    def hidden(self) -> torch.Tensor:
        """[B, gamma-1, H] bf16 drafter hidden states (confidence-head workload)."""
        if "hidden" not in self._cache:
            wl = self.wl
            w = self.head_w.astype(np.float64)
            out = np.empty((self.B, wl.G1, wl.head_H), np.float32)
            for b in range(self.B):
                r = self._rng(b, self._CONF)
                c = self.cls(b)
                ct = r.beta(c.a, c.b, size=wl.G1)
                z = np.log(ct) - np.log1p(-ct)
                gz = r.standard_normal((wl.G1, wl.head_H))
                gz = gz + ((z - gz @ w - float(self.head_b)) / (w @ w))[:, None] * w[None, :]
                out[b] = gz
            self._cache["hidden"] = _round(out, "bf16")
        return self._cache["hidden"]

    def cost_tables(self):
        """(bias, alpha [B+1], theta [B*gamma+1]) float32 milliseconds."""
        wl = self.wl
        alpha = np.zeros(self.B + 1, np.float32)
        theta = (np.float32(wl.theta_ms_per_token) * np.arange(self.B * wl.gamma + 1, dtype=np.float32)).astype(np.float32)
        return np.float32(wl.bias_ms), alpha, theta

    # ------------------------------------------------------------------ stage 2-3 inputs
    def request_qkv(self, b: int):
        """q [gamma, Hq, D], k_new / v_new [gamma, Hkv, D] for every block position."""
        wl = self.wl
        r = self._rng(b, self._QKV)
        q = r.standard_normal((wl.gamma, wl.Hq, wl.D), dtype=np.float32)
        k = r.standard_normal((wl.gamma, wl.Hkv, wl.D), dtype=np.float32)
        v = r.standard_normal((wl.gamma, wl.Hkv, wl.D), dtype=np.float32)
        return _round(q, wl.kv_dtype), _round(k, wl.kv_dtype), _round(v, wl.kv_dtype)

    def request_context_kv(self, b: int):
        """Cached context K, V of request b: [L_b, Hkv, D] each, in position order."""
        wl = self.wl
        r = self._rng(b, self._CTX)
        L = int(self.context_lens[b])
        K = r.standard_normal((L, wl.Hkv, wl.D), dtype=np.float32)
        V = r.standard_normal((L, wl.Hkv, wl.D), dtype=np.float32)
        return _round(K, wl.kv_dtype), _round(V, wl.kv_dtype)

    def request_pack_src(self, b: int) -> torch.Tensor:
        r = self._rng(b, self._PACK)
        return _round(r.standard_normal((self.wl.gamma, self.wl.pack_hidden), dtype=np.float32), "bf16")

    # ------------------------------------------------------------------ stage 4-5 inputs
    def request_logits(self, b: int):
        """target [gamma, V], draft [gamma-1, V] (logit dtype), draft tokens [gamma-1]."""
        wl = self.wl
        r = self._rng(b, self._LOGITS)
        t = r.standard_normal((wl.gamma, wl.V), dtype=np.float32) * np.float32(wl.target_logit_std)
        noise = r.standard_normal((wl.G1, wl.V), dtype=np.float32) * draft_sigma(self.conf64(b))[:, None]
        d = t[:-1] + noise
        tt, dd = _round(t, wl.logit_dtype), _round(d, wl.logit_dtype)
        # Gumbel-max draw of each draft token from softmax(draft row), float64
        rg = self._rng(b, self._GUMBEL)
        d64 = dd.to(torch.float64).numpy()
        gum = -np.log(-np.log(rg.random((wl.G1, wl.V))))
        tokens = np.argmax(d64 + gum, axis=1).astype(np.int32)
        return tt, dd, tokens

    def request_uniforms(self, b: int):
        r = self._rng(b, self._UNIF)
        return r.random(self.wl.G1, dtype=np.float32), np.float32(r.random(dtype=np.float32))

    def uniforms(self):
        ua = np.empty((self.B, self.wl.G1), np.float32)
        ur = np.empty(self.B, np.float32)
        for b in range(self.B):
            ua[b], ur[b] = self.request_uniforms(b)
        return ua, ur


def v_block(page: int) -> int:
    """Column-block width of the V cache layout (32 slots, or the page if not a multiple of 32)."""
    return 32 if page % 32 == 0 else page


def paged_cache(inp: Inputs, fill_unused=float("nan"), requests=None):
    """Host page pools in the library's layout, filled with each request's context.

    k_pool [num_pages, Hkv, page, D] (element (page, g, slot, d)), v_pool
    [num_pages, Hkv, page // VB, D, VB] (element (page, g, slot // VB, d, slot % VB), VB = 32
    when page is a multiple of 32, else the page).  Slots that hold no context
    position (the tail of each request's last pages) are set to ``fill_unused`` so that a
    kernel reading them would be noticed.  ``requests`` limits the fill to a subset.
    """
    wl = inp.wl
    dt = _TORCH[wl.kv_dtype]
    P = inp.num_pages
    k_pool = torch.full((P, wl.Hkv, wl.page, wl.D), fill_unused, dtype=dt)
    VB = v_block(wl.page)
    v_pool = torch.full((P, wl.Hkv, wl.page // VB, wl.D, VB), fill_unused, dtype=dt)
    reqs = range(inp.B) if requests is None else requests
    for b in reqs:
        K, V = inp.request_context_kv(b)
        L = int(inp.context_lens[b])
        for j in range(-(-L // wl.page)):
            pg = int(inp.block_table[b, j])
            lo, hi = j * wl.page, min(L, (j + 1) * wl.page)
            k_pool[pg, :, : hi - lo, :] = K[lo:hi].permute(1, 0, 2)
            for s0 in range(lo, hi, VB):
                s1 = min(hi, s0 + VB)
                v_pool[pg, :, (s0 - lo) // VB, :, : s1 - s0] = V[s0:s1].permute(1, 2, 0)
    return k_pool, v_pool


def calibration_trace(seed: int, N: int, G1: int, T_true, beta=(6.0, 1.5), noise: float = 0.0,
                      censor: bool = False):
    """Synthetic acceptance trace with a known head temperature (recipe in the module
    docstring).  Returns (z float32 [N, G1], accept_len int32 [N], observed_len int32 [N])."""
    ss = np.random.SeedSequence([seed, 0xCA1])
    r_q, r_z, r_u, r_o = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4))
    T = np.broadcast_to(np.asarray(T_true, dtype=np.float64), (G1,))
    q = r_q.beta(beta[0], beta[1], size=(N, G1))
    q = np.clip(q, 1e-12, 1 - 1e-12)
    z = (T[None, :] * np.log(q / (1.0 - q)) + noise * r_z.standard_normal((N, G1))).astype(np.float32)
    acc = r_u.random((N, G1)) < q
    n = np.where(acc.all(axis=1), G1, np.argmin(acc, axis=1)).astype(np.int32)
    obs = r_o.integers(0, G1 + 1, size=N).astype(np.int32) if censor else np.full(N, G1, np.int32)
    return z, n, obs


def markov_inputs(seed: int, B: int, G1: int, V: int, r: int = 256, dtype: str = "bf16"):
    """Inputs of the Markov sequential head (recipe in the module docstring).  Returns dict
    U (torch [B, G1, V]), anchor int32 [B], u float32 [B, G1], q1, q2 int8 [V, r],
    s1, s2 float32 [V]."""
    ss = np.random.SeedSequence([seed, 0x3A4])
    rU, rA, rW, rS = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4))
    U = _round(2.0 * rU.standard_normal((B, G1, V), dtype=np.float32), dtype)
    anchor = rA.integers(0, V, size=B).astype(np.int32)
    u = rA.random((B, G1), dtype=np.float32)
    q1 = rW.integers(-127, 128, size=(V, r), dtype=np.int8)
    q2 = rW.integers(-127, 128, size=(V, r), dtype=np.int8)
    s1 = (4.2e-3 * rS.uniform(0.5, 1.5, size=V)).astype(np.float32)
    s2 = (4.2e-3 * rS.uniform(0.5, 1.5, size=V)).astype(np.float32)
    return {"U": U, "anchor": anchor, "u": u, "q1": q1, "q2": q2, "s1": s1, "s2": s2}
