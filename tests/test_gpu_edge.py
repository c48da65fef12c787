"""GPU edge cases through the C ABI, each against the oracle.

Covers shapes the five workloads do not reach: scheduler candidate counts on both ordering
paths (the one-workgroup merge up to 1024 candidates; the ranking spread over one workgroup
per request beyond, with 2 and 4 keys a thread after it), heavy survival ties, the confidence head
with per-position temperatures (bf16 and f32 hidden states), single-draft and
single-request batches, acceptance batches whose windows are all 1 (no drafts: every
request takes the bonus draw) or all gamma, cap-accept with caps of 1, random and the whole
block, odd and very large vocabularies, and packs of rows whose size is not a multiple of
16 bytes.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ragged_verify_acceptance_amd import rva

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _schedule_case(B, gamma, conf, theta_per_token, static=False):
    G = gamma - 1
    conf = np.asarray(conf, np.float32).reshape(B, G)
    alpha = np.zeros(B + 1, np.float32)
    theta = (np.float32(theta_per_token) * np.arange(B * gamma + 1, dtype=np.float32)).astype(np.float32)
    bias = np.float32(20.0)
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    conf_out = torch.empty((B, G), dtype=torch.float32, device=DEV)
    surv = torch.empty((B, G), dtype=torch.float32, device=DEV)
    windows = torch.empty(B, dtype=torch.int32, device=DEV)
    K = torch.empty(1, dtype=torch.int32, device=DEV)
    ratio = torch.empty(1, dtype=torch.float64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.schedule_windows(B, gamma, 1 if static else 0, None, 0, None, 0.0, t(conf), None,
                         float(bias), t(alpha), t(theta), conf_out, surv, windows, K, ratio,
                         status)
    torch.cuda.synchronize()
    a = oracle.survival(conf)
    ref = oracle.schedule_windows(a, gamma, bias, alpha, theta, static=static)
    assert np.array_equal(conf_out.cpu().numpy().view(np.uint32), conf.view(np.uint32))
    assert np.array_equal(surv.cpu().numpy().view(np.uint32), a.view(np.uint32))
    if not ref["near_tie"]:
        assert np.array_equal(windows.cpu().numpy(), ref["windows"])
        assert int(K.item()) == ref["K"]
    assert abs(float(ratio.item()) - ref["ratio"]) <= 1e-12 * abs(ref["ratio"])
    assert int(status.item()) == 0
    return ref


@pytest.mark.parametrize("B,gamma", [(1, 2), (3, 5), (64, 17), (128, 16), (200, 8), (256, 16),
                                     (64, 64), (2048, 2), (4096, 2), (1100, 3)])
@pytest.mark.parametrize("kind", ["beta", "ties"])
def test_schedule_sizes(B, gamma, kind):
    """Candidate counts 1 .. 4096 (every ordering path and keys-a-thread layout; runs of one
    draft on the ranked path), with and without ties."""
    print(f"[schedule-size] B={B} gamma={gamma} {kind}", flush=True)
    rng = np.random.default_rng(B * 100 + gamma)
    G = gamma - 1
    if kind == "beta":
        conf = rng.beta(6.0, 1.5, size=(B, G))
    else:  # few distinct values: long runs of equal survival across requests
        conf = rng.choice([1.0, 0.875, 0.75, 0.5], size=(B, G))
    for theta in (0.01, 0.19, 2.0):
        _schedule_case(B, gamma, conf, theta)
    _schedule_case(B, gamma, conf, 0.19, static=True)


def _accept_case(B, gamma, V, windows, seed, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    G1 = gamma - 1
    windows = np.asarray(windows, np.int64)
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    M = int(cu[-1])
    max_rows = M + 3
    tl = (rng.standard_normal((max_rows, V)) * 2.0).astype(np.float32)
    dl = (rng.standard_normal((B * G1, V)) * 2.0).astype(np.float32)
    # drafts close to the target rows for half the requests (high acceptance)
    for b in range(B):
        for k in range(windows[b] - 1):
            if b % 2 == 0:
                dl[b * G1 + k] = tl[cu[b] + k] + 0.3 * rng.standard_normal(V).astype(np.float32)
    tl_t = torch.from_numpy(tl).to(dtype)
    dl_t = torch.from_numpy(dl).to(dtype)
    tokens = rng.integers(0, V, size=(B, G1)).astype(np.int32)
    ua = rng.random((B, G1)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ctx0 = rng.integers(10, 100, size=B).astype(np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    com = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
    ctx = d(ctx0)
    pt = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    pd = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    lab = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, max_rows), dtype=torch.uint8, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.accept_and_commit(B, gamma, V, max_rows, tl_t.to(DEV), dl_t.to(DEV), d(tokens), d(ua),
                          d(ur), d(cu), acc, com, ctx, pt, pd, lab, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    tl64 = tl_t.double().numpy()
    dl64 = dl_t.double().numpy()
    acc_h, com_h, ctx_h = acc.cpu().numpy(), com.cpu().numpy(), ctx.cpu().numpy()
    lab_h = lab.cpu().numpy()
    flips = 0
    for b in range(B):
        w = int(windows[b])
        r = oracle.accept_request(tl64[cu[b]:cu[b] + w], dl64[b * G1:b * G1 + w - 1],
                                  tokens[b, : w - 1], ua[b, : w - 1], ur[b])
        band = any(m < 1e-6 for m in r["margins"]) or r["draw_margin"] < 1e-9
        same = acc_h[b] == r["n"] and list(com_h[b, : r["n"] + 1]) == list(r["committed"])
        if not same:
            assert band, f"request {b}: {acc_h[b]} {com_h[b]} vs {r['n']} {r['committed']}"
            flips += 1
            continue
        assert np.all(com_h[b, r["n"] + 1:] == -1)
        assert ctx_h[b] == ctx0[b] + r["n"] + 1
        np.testing.assert_allclose(lab_h[b, : w - 1], r["labels"], atol=1e-5, rtol=0)
        assert np.all(np.isnan(lab_h[b, w - 1:]))
    assert flips <= 1


@pytest.mark.parametrize("case", ["all-bonus", "all-full", "mixed", "one-request"])
def test_accept_edges(case):
    print(f"[accept-edge] {case}", flush=True)
    V = 50_000  # not a multiple of the 16384-entry segment: a ragged last segment
    if case == "all-bonus":
        _accept_case(8, 6, V, [1] * 8, seed=1)
    elif case == "all-full":
        _accept_case(8, 6, V, [6] * 8, seed=2)
    elif case == "mixed":
        _accept_case(16, 9, V, [1, 9, 2, 8, 3, 7, 4, 6, 5, 5, 1, 9, 2, 2, 9, 1], seed=3)
    else:
        _accept_case(1, 4, V, [4], seed=4)


@pytest.mark.parametrize("V", [1000, 16384, 16391])
def test_accept_odd_vocab(V):
    """Vocabulary sizes below, at and just past one segment; 16391 is not a multiple of 8,
    so the unaligned load paths run."""
    print(f"[accept-vocab] V={V}", flush=True)
    _accept_case(6, 5, V, [5, 1, 3, 4, 2, 5], seed=V)
    _accept_case(6, 5, V, [5, 1, 3, 4, 2, 5], seed=V + 1, dtype=torch.float32)


def test_accept_vocab_beyond_one_wave_of_segments():
    """V = 1,100,000: 68 segments of 16384, more than one wave's 64 lanes, so the pick's
    segment search takes its general path (segment sums re-read per step) and the
    normaliser loops stride over the segments."""
    print("[accept-vocab] V=1100000", flush=True)
    _accept_case(3, 3, 1_100_000, [3, 1, 2], seed=11)


@pytest.mark.parametrize("elems,dtype", [(3, torch.bfloat16), (2050, torch.bfloat16), (5, torch.float32),
                                         (20001, torch.bfloat16), (151936, torch.bfloat16)],
                         ids=["6-byte-rows", "4100-byte-rows", "20-byte-rows", "40002-byte-rows",
                              "303872-byte-rows"])
def test_pack_unaligned_rows(elems, dtype):
    """Row sizes that are not multiples of 16 bytes take the scalar copy path, and rows above
    16 KB are cut into column parts (40002 bytes: three parts on the scalar path; a
    vocabulary-wide bf16 logits row: 19 parts on the vector path); the total 14 rounds up
    to tier 16 (two zero rows); rows past the tier keep their contents."""
    print(f"[pack-edge] {elems} x {dtype}", flush=True)
    rng = np.random.default_rng(elems)
    B, gamma = 5, 4
    windows = np.array([1, 4, 2, 3, 4], np.int32)
    ctx = rng.integers(0, 1000, size=B).astype(np.int32)
    tiers = [8, 12, 16, 20]
    max_rows = 20
    src = torch.from_numpy(rng.standard_normal((B, gamma, elems)).astype(np.float32)).to(dtype)
    ref = oracle.pack_ragged(windows, ctx, tiers, src=src.double().numpy(), max_rows=max_rows)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    dst = torch.full((max_rows, elems), 7.0, dtype=dtype, device=DEV)
    cu = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    row_req = torch.empty(max_rows, dtype=torch.int32, device=DEV)
    row_pos = torch.empty(max_rows, dtype=torch.int32, device=DEV)
    tt = torch.empty(2, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.pack_ragged(B, gamma, d(windows), d(ctx), tiers, src.to(DEV), dst, max_rows, cu, row_req,
                    row_pos, tt, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    M, tier = ref["M"], ref["tier"]
    assert (M, tier) == (14, 16) and tt.cpu().tolist() == [M, tier]
    assert cu.cpu().tolist() == list(ref["cu_seqlens"])
    assert row_req.cpu().tolist() == list(ref["row_req"])
    assert row_pos.cpu().tolist() == list(ref["row_pos"])
    got = dst.double().cpu().numpy()
    assert np.array_equal(got[:tier], ref["dst"][:tier])
    assert np.all(got[tier:] == 7.0)


@pytest.mark.parametrize("cap_kind", ["all-1", "random", "all-gamma"])
def test_accept_capped_edges(cap_kind):
    """Cap-accept with caps of 1 (only the anchor's bonus draw may be committed), random
    caps, and caps equal to the block (plain static acceptance), against the oracle."""
    print(f"[accept-capped-edge] {cap_kind}", flush=True)
    rng = np.random.default_rng({"all-1": 21, "random": 22, "all-gamma": 23}[cap_kind])
    B, gamma, V = 12, 6, 40_000
    G1 = gamma - 1
    caps = {"all-1": np.ones(B, np.int32), "all-gamma": np.full(B, gamma, np.int32),
            "random": rng.integers(1, gamma + 1, size=B).astype(np.int32)}[cap_kind]
    cu = (np.arange(B + 1) * gamma).astype(np.int32)  # whole blocks verified
    max_rows = B * gamma + 2
    tl = (rng.standard_normal((max_rows, V)) * 2.0).astype(np.float32)
    dl = (rng.standard_normal((B * G1, V)) * 2.0).astype(np.float32)
    for b in range(0, B, 2):  # drafts close to the target for half the requests
        for k in range(G1):
            dl[b * G1 + k] = tl[cu[b] + k] + 0.3 * rng.standard_normal(V).astype(np.float32)
    tl_t = torch.from_numpy(tl).to(torch.bfloat16)
    dl_t = torch.from_numpy(dl).to(torch.bfloat16)
    tokens = rng.integers(0, V, size=(B, G1)).astype(np.int32)
    ua = rng.random((B, G1)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ctx0 = rng.integers(10, 100, size=B).astype(np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    full = torch.empty(B, dtype=torch.int32, device=DEV)
    com = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
    ctx = d(ctx0)
    pt = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    pd = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    lab = torch.empty((B, G1), dtype=torch.float32, device=DEV)
    ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, max_rows), dtype=torch.uint8, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.accept_capped(B, gamma, V, max_rows, tl_t.to(DEV), dl_t.to(DEV), d(tokens), d(ua), d(ur),
                      d(cu), d(caps), acc, full, com, ctx, pt, pd, lab, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    tl64, dl64 = tl_t.double().numpy(), dl_t.double().numpy()
    acc_h, full_h, com_h, ctx_h, lab_h = (x.cpu().numpy() for x in (acc, full, com, ctx, lab))
    flips = 0
    for b in range(B):
        r = oracle.accept_request_capped(tl64[cu[b]:cu[b] + gamma], dl64[b * G1:(b + 1) * G1],
                                         tokens[b], ua[b], ur[b], int(caps[b]))
        band = any(m < 1e-6 for m in r["margins"]) or r["draw_margin"] < 1e-9
        same = acc_h[b] == r["n"] and full_h[b] == r["n_full"] and \
            list(com_h[b, : r["n"] + 1]) == list(r["committed"])
        if not same:
            assert band, f"request {b}: {acc_h[b]}/{full_h[b]} {com_h[b]} vs {r['n']}/{r['n_full']} {r['committed']}"
            flips += 1
            continue
        assert np.all(com_h[b, r["n"] + 1:] == -1)
        assert ctx_h[b] == ctx0[b] + r["n"] + 1
        assert acc_h[b] <= caps[b] - 1
        np.testing.assert_allclose(lab_h[b], r["labels"], atol=1e-5, rtol=0)
    assert flips <= 1


@pytest.mark.parametrize("hdtype", [torch.bfloat16, torch.float32], ids=["bf16-hidden", "f32-hidden"])
def test_schedule_head_with_temperatures(hdtype):
    """The confidence head with per-position temperatures (c = sigmoid(z / T_k)) feeding the
    window choice, against the oracle: confidences and survival bit-exact, windows exact
    unless the oracle flags a near tie."""
    print(f"[schedule-head-T] {hdtype}", flush=True)
    rng = np.random.default_rng(31)
    B, gamma, H = 24, 7, 640
    G = gamma - 1
    hidden = torch.from_numpy((rng.standard_normal((B, G, H)) * 0.5).astype(np.float32)).to(hdtype)
    head_w = (rng.standard_normal(H) * 0.08).astype(np.float32)
    head_b = np.float32(1.2)
    T = np.array([0.7, 1.0, 1.3, 1.9, 2.5, 4.0], np.float32)
    alpha = np.zeros(B + 1, np.float32)
    theta = (np.float32(0.19) * np.arange(B * gamma + 1, dtype=np.float32)).astype(np.float32)
    bias = np.float32(20.0)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    conf_out = torch.empty((B, G), dtype=torch.float32, device=DEV)
    surv = torch.empty((B, G), dtype=torch.float32, device=DEV)
    windows = torch.empty(B, dtype=torch.int32, device=DEV)
    K = torch.empty(1, dtype=torch.int32, device=DEV)
    ratio = torch.empty(1, dtype=torch.float64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.schedule_windows(B, gamma, 0, hidden.to(DEV), H, d(head_w), float(head_b), None, d(T),
                         float(bias), d(alpha), d(theta), conf_out, surv, windows, K, ratio, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    c = oracle.confidence_from_head(hidden.double().numpy(), head_w, head_b, T)
    a = oracle.survival(c)
    ref = oracle.schedule_windows(a, gamma, bias, alpha, theta)
    assert np.array_equal(conf_out.cpu().numpy().view(np.uint32), c.view(np.uint32))
    assert np.array_equal(surv.cpu().numpy().view(np.uint32), a.view(np.uint32))
    if not ref["near_tie"]:
        assert np.array_equal(windows.cpu().numpy(), ref["windows"])
        assert int(K.item()) == ref["K"]


def test_accept_without_optional_outputs():
    """Acceptance with no labels and no probability outputs (the pair pass then runs only
    its draw slots) commits exactly what the full call commits on the same inputs."""
    print("[accept-optional] labels/probs off", flush=True)
    rng = np.random.default_rng(41)
    B, gamma, V = 16, 8, 30_000
    G1 = gamma - 1
    windows = rng.integers(1, gamma + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    max_rows = int(cu[-1]) + 2
    tl = (rng.standard_normal((max_rows, V)) * 2.0).astype(np.float32)
    dl = (rng.standard_normal((B * G1, V)) * 2.0).astype(np.float32)
    for b in range(0, B, 2):
        for k in range(windows[b] - 1):
            dl[b * G1 + k] = tl[cu[b] + k] + 0.3 * rng.standard_normal(V).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    tl_d = torch.from_numpy(tl).to(torch.bfloat16).to(DEV)
    dl_d = torch.from_numpy(dl).to(torch.bfloat16).to(DEV)
    tokens = d(rng.integers(0, V, size=(B, G1)).astype(np.int32))
    ua = d(rng.random((B, G1)).astype(np.float32))
    ur = d(rng.random(B).astype(np.float32))
    ctx0 = rng.integers(10, 100, size=B).astype(np.int32)
    ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, max_rows), dtype=torch.uint8, device=DEV)
    runs = []
    for full_outputs in (True, False):
        acc = torch.empty(B, dtype=torch.int32, device=DEV)
        com = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
        ctx = d(ctx0)
        opt = [torch.empty((B, G1), dtype=torch.float32, device=DEV) if full_outputs else None
               for _ in range(3)]
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        rva.accept_and_commit(B, gamma, V, max_rows, tl_d, dl_d, tokens, ua, ur, d(cu), acc, com, ctx,
                              opt[0], opt[1], opt[2], ws, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        runs.append((acc.cpu().numpy(), com.cpu().numpy(), ctx.cpu().numpy()))
    for x, y in zip(runs[0], runs[1]):
        assert np.array_equal(x, y)
