"""GPU parity of rva_verify_attention on shapes the five workloads do not reach.

Each case builds a small seeded batch and compares the HIP path with the oracle
(``oracle.verify_attention``, float64 on the same bf16/f32-rounded inputs):

* head dimension 64 on the fast path (bf16), GQA groups of 1, 4 and 8, page sizes 32, 128
  and 256;
* the generic path: float32 at pages of 16, 24 and 32 (contexts of several 256-key passes),
  bf16 at a page of 48 slots, at window x group above 64 columns and at 1030 requests;
* column blocks NB = 1, 2 and 4 (window rows x group of 16, 32 and 64 columns);
* contexts of 0, 1, one short of / exactly / one past a 32-key tile and of a page;
* batches whose weighted work is below the grid size, and one long segment spread over
  every workgroup.

Bar: max over (row, head) of max|o - r| / max|r| <= 1e-2 for bf16 (1e-4 for float32, whose
output is not rounded to 8 bits); pad rows [M, tier) zero and rows
past the tier untouched; both caches after the call (the appended window K/V and every
other entry) bit-identical to the oracle's; device status 0.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import default_scale, v_block
from ragged_verify_acceptance_amd import rva

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATTN_TOL = 1e-2
ATTN_TOL_F32 = 1e-4

# name, kv dtype, D, Hq, Hkv, page size, context lengths, windows
CASES = [
    ("d64-g4-p32-nb1", "bf16", 64, 8, 2, 32, [0, 1, 31, 33, 100], [1, 4, 2, 3, 4]),
    ("d64-g8-p128-nb4", "bf16", 64, 16, 2, 128, [5, 127, 128, 300], [8, 1, 6, 8]),
    ("d128-g1-p256-nb1", "bf16", 128, 8, 8, 256, [0, 5, 255, 256, 700], [16, 3, 1, 9, 16]),
    ("d128-g4-p32-nb2", "bf16", 128, 16, 4, 32, [31, 32, 63, 64, 257, 1000], [8, 7, 1, 5, 8, 2]),
    ("d128-f32-p16-generic", "f32", 128, 4, 2, 16, [0, 17, 40], [3, 1, 4]),
    # generic path: several passes of 256 keys per column, 32-slot V blocks, float32
    ("d64-f32-p32-generic-long", "f32", 64, 8, 2, 32, [3000, 0, 700, 255, 256], [5, 2, 7, 1, 3]),
    # generic path: group 1, page of 24 slots (not a power of two), contexts around a page
    ("d64-f32-p24-generic-g1", "f32", 64, 4, 4, 24, [0, 23, 24, 25, 500], [2, 6, 1, 3, 6]),
    # generic path in bf16: a page of 48 slots, and window x group = 80 columns (> 64)
    ("d64-bf16-p48-generic", "bf16", 64, 8, 2, 48, [47, 48, 200, 1000], [3, 1, 4, 2]),
    ("d128-bf16-wide-generic", "bf16", 128, 32, 2, 64, [100, 2000, 0], [5, 3, 4]),
    # generic path in bf16: more requests than the MFMA path's table holds (1030 > 1024),
    # and more (request, column) pairs (16480) than the capped grid has workgroups per row
    ("d128-bf16-b1030-generic", "bf16", 128, 16, 4, 64,
     [int(x) for x in np.random.default_rng(1030).integers(0, 300, 1030)],
     [int(x) for x in np.random.default_rng(1031).integers(1, 5, 1030)]),
    # one segment over every workgroup (the merge's loop over more than four shares)
    ("d128-g4-p64-one-long", "bf16", 128, 4, 1, 64, [20000], [3]),
    ("d64-g16-p64-nb4", "bf16", 64, 32, 2, 64, [700, 33, 2000], [4, 2, 3]),
    ("d64-g2-p32-nb2", "bf16", 64, 4, 2, 32, [1000, 64, 5], [16, 9, 12]),
    # more work units than workgroups at D = 64: segments cut between two or three shares
    ("d64-g4-p64-long-nb1", "bf16", 64, 8, 2, 64, [4000, 3100, 5000, 2500, 4100, 3999, 4500, 3000],
     [4, 1, 3, 4, 2, 4, 1, 3]),
    ("d64-g8-p64-long-nb4", "bf16", 64, 16, 2, 64, [3000, 4096, 2048, 5000], [8, 6, 2, 7]),
    # one kv head for all query heads (group 32), and pages of 1024 slots
    ("d128-mqa-g32-p64", "bf16", 128, 32, 1, 64, [500, 3000, 7], [2, 1, 2]),
    ("d128-g4-p1024", "bf16", 128, 16, 4, 1024, [1023, 1024, 2500, 0], [8, 3, 5, 8]),
]


def _round(x, dtype):
    """float64 values of x rounded to the kv dtype (bf16: via float32, nearest even)."""
    t = torch.from_numpy(np.asarray(x, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_shape(case):
    name, dtype, D, Hq, Hkv, P, Ls, ws = case
    print(f"[attention shape] {name}", flush=True)
    rng = np.random.default_rng(sum(ord(ch) for ch in name))
    B = len(Ls)
    max_w = max(ws)
    VB = v_block(P)
    pages_per = [-(-(L + max_w) // P) for L in Ls]
    max_pages = max(pages_per)
    num_pages = sum(pages_per) + 3
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.zeros((B, max_pages), np.int32)
    o = 0
    for b in range(B):
        bt[b, : pages_per[b]] = perm[o: o + pages_per[b]]
        o += pages_per[b]
    cu = np.concatenate([[0], np.cumsum(ws)]).astype(np.int32)
    M = int(cu[-1])
    tier = M + 2
    max_rows = tier + 1

    q_t = _round(rng.standard_normal((max_rows, Hq, D)), dtype)
    kn_t = _round(rng.standard_normal((max_rows, Hkv, D)), dtype)
    vn_t = _round(rng.standard_normal((max_rows, Hkv, D)), dtype)
    kc_t = _round(rng.standard_normal((num_pages, Hkv, P, D)), dtype)
    vc_t = _round(rng.standard_normal((num_pages, Hkv, P // VB, D, VB)), dtype)
    scale = default_scale(D)

    ref, kc_ref, vc_ref = oracle.verify_attention(
        q_t.double().numpy(), kn_t.double().numpy(), vn_t.double().numpy(),
        kc_t.double().numpy(), vc_t.double().numpy(), bt, np.asarray(Ls), cu, tier, scale)

    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    q, kn, vn = q_t.to(DEV), kn_t.to(DEV), vn_t.to(DEV)
    kc, vc = kc_t.clone().to(DEV), vc_t.clone().to(DEV)
    out = torch.full((max_rows, Hq, D), float("nan"), dtype=q.dtype, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvd = rva.BF16 if dtype == "bf16" else rva.F32
    wsz = rva.verify_attention_workspace_size(B, max_w, Hq, Hkv, D, P, max_pages, kvd)
    ws_buf = torch.empty(max(wsz, 256), dtype=torch.uint8, device=DEV)
    rva.verify_attention(B, max_w, max_rows, Hq, Hkv, D, P, num_pages, max_pages, q, kn, vn, kc,
                         vc, t(bt), t(np.asarray(Ls, np.int32)), t(cu),
                         t(np.array([M, tier], np.int32)), float(scale), out, ws_buf, status)
    torch.cuda.synchronize()

    assert int(status.item()) == 0
    o_h = out.double().cpu().numpy()
    err = 0.0
    for r in range(M):
        for h in range(Hq):
            den = np.max(np.abs(ref[r, h]))
            err = max(err, np.max(np.abs(o_h[r, h] - ref[r, h])) / den)
    print(f"[attention shape] {name}: max rel err {err:.2e}", flush=True)
    assert err <= (ATTN_TOL if dtype == "bf16" else ATTN_TOL_F32)
    assert np.all(o_h[M:tier] == 0.0)
    assert np.all(np.isnan(o_h[tier:]))
    assert np.array_equal(kc.double().cpu().numpy(), kc_ref)
    assert np.array_equal(vc.double().cpu().numpy(), vc_ref)
