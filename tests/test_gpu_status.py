"""Device-side data errors: the status bits, and the unaffected requests still exact.

Each case feeds one bad value that the kernels' own checks catch before any access uses
it (the entry points only validate host-side scalars): the kernel ORs a RVA_DEV_* bit into
device_status, clamps or skips the bad item so every access stays in bounds, and the
other requests' results must equal the oracle's.
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
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _attention_batch(seed, Ls, ws, D=128, Hq=8, Hkv=2, P=64):
    rng = np.random.default_rng(seed)
    B = len(Ls)
    max_w = max(ws)
    VB = v_block(P)
    pages_per = [-(-(L + max_w) // P) for L in Ls]
    max_pages = max(pages_per)
    num_pages = sum(pages_per) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.zeros((B, max_pages), np.int32)
    o = 0
    for b in range(B):
        bt[b, : pages_per[b]] = perm[o: o + pages_per[b]]
        o += pages_per[b]
    cu = np.concatenate([[0], np.cumsum(ws)]).astype(np.int32)
    M = int(cu[-1])
    rows = M + 2
    bf = lambda shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    t = dict(q=bf((rows, Hq, D)), kn=bf((rows, Hkv, D)), vn=bf((rows, Hkv, D)),
             kc=bf((num_pages, Hkv, P, D)), vc=bf((num_pages, Hkv, P // VB, D, VB)))
    return dict(B=B, D=D, Hq=Hq, Hkv=Hkv, P=P, max_w=max_w, max_pages=max_pages,
                num_pages=num_pages, bt=bt, cu=cu, M=M, rows=rows, Ls=np.asarray(Ls, np.int32), **t)


def _run_attention(x, bt, Ls):
    kc, vc = x["kc"].clone().to(DEV), x["vc"].clone().to(DEV)
    out = torch.zeros((x["rows"], x["Hq"], x["D"]), dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    wsz = rva.verify_attention_workspace_size(x["B"], x["max_w"], x["Hq"], x["Hkv"], x["D"], x["P"],
                                              x["max_pages"], rva.BF16)
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=DEV)
    rva.verify_attention(x["B"], x["max_w"], x["rows"], x["Hq"], x["Hkv"], x["D"], x["P"],
                         x["num_pages"], x["max_pages"], x["q"].to(DEV), x["kn"].to(DEV),
                         x["vn"].to(DEV), kc, vc, d(bt), d(Ls), d(x["cu"]),
                         d(np.array([x["M"], x["M"] + 1], np.int32)),
                         float(default_scale(x["D"])), out, ws, status)
    torch.cuda.synchronize()
    return int(status.item()), out.double().cpu().numpy(), kc.double().cpu().numpy()


def _oracle_attention(x, Ls):
    return oracle.verify_attention(x["q"].double().numpy(), x["kn"].double().numpy(),
                                   x["vn"].double().numpy(), x["kc"].double().numpy(),
                                   x["vc"].double().numpy(), x["bt"], Ls, x["cu"], x["M"] + 1,
                                   default_scale(x["D"]))


def _rel_err(o, r):
    return float(np.max(np.max(np.abs(o - r), axis=-1) / np.max(np.abs(r), axis=-1)))


# page 64: the MFMA path; page 48 (not a power of two): the generic path
PATHS = pytest.mark.parametrize("P", [64, 48], ids=["mfma", "generic"])


@PATHS
def test_attention_bad_page_entry(P):
    """A block-table entry past the pool: RVA_DEV_BAD_PAGE; that request's keys in the page
    are replaced (MFMA path: page 0) or left out (generic path), every other request is
    exact, and the window appends (in valid pages) land."""
    print(f"[status] attention bad page, page {P}", flush=True)
    x = _attention_batch(51, [300, 700, 90, 500], [3, 4, 2, 4], P=P)
    bt = x["bt"].copy()
    bt[1, 0] = x["num_pages"] + 5  # request 1, positions 0..63
    st, out, kc = _run_attention(x, bt, x["Ls"])
    assert st & rva.DEV_BAD_PAGE
    ref, kc_ref, _ = _oracle_attention(x, x["Ls"])
    for b in (0, 2, 3):
        r0, r1 = x["cu"][b], x["cu"][b + 1]
        assert _rel_err(out[r0:r1], ref[r0:r1]) <= 1e-2
    assert np.array_equal(kc, kc_ref)


@PATHS
def test_attention_context_past_page_table(P):
    """A context that does not fit its page-table row: RVA_DEV_BAD_CONTEXT; the request is
    skipped (no attention, no append), the others are exact."""
    print(f"[status] attention bad context, page {P}", flush=True)
    x = _attention_batch(52, [300, 700, 90, 500], [3, 4, 2, 4], P=P)
    Ls = x["Ls"].copy()
    Ls[2] = x["max_pages"] * x["P"]  # L + w beyond the row
    st, out, _ = _run_attention(x, x["bt"], Ls)
    assert st & rva.DEV_BAD_CONTEXT
    ref, _, _ = _oracle_attention(x, x["Ls"])
    for b in (0, 1, 3):
        r0, r1 = x["cu"][b], x["cu"][b + 1]
        assert _rel_err(out[r0:r1], ref[r0:r1]) <= 1e-2


def test_accept_token_out_of_range():
    """Draft tokens -1 and V: RVA_DEV_BAD_TOKEN, and the kernels use the clamped ids 0 and
    V - 1 -- the oracle given those ids agrees on every request."""
    print("[status] accept bad tokens", flush=True)
    rng = np.random.default_rng(53)
    B, gamma, V = 6, 5, 20_000
    G1 = gamma - 1
    windows = np.array([5, 3, 5, 2, 4, 5])
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    max_rows = int(cu[-1]) + 1
    tl = torch.from_numpy((rng.standard_normal((max_rows, V)) * 2.0).astype(np.float32)).to(torch.bfloat16)
    dlv = (rng.standard_normal((B * G1, V)) * 2.0).astype(np.float32)
    for b in range(B):
        for k in range(windows[b] - 1):
            dlv[b * G1 + k] = tl[cu[b] + k].float().numpy() + 0.2 * rng.standard_normal(V).astype(np.float32)
    dl = torch.from_numpy(dlv).to(torch.bfloat16)
    tokens = rng.integers(0, V, size=(B, G1)).astype(np.int32)
    tokens[0, 0] = -1
    tokens[2, 1] = V
    ua = rng.random((B, G1)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ctx0 = np.full(B, 50, np.int32)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    com = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
    ctx = d(ctx0)
    ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, max_rows), dtype=torch.uint8, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.accept_and_commit(B, gamma, V, max_rows, tl.to(DEV), dl.to(DEV), d(tokens), d(ua), d(ur),
                          d(cu), acc, com, ctx, None, None, None, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) & rva.DEV_BAD_TOKEN
    clamped = np.clip(tokens, 0, V - 1)
    acc_h, com_h = acc.cpu().numpy(), com.cpu().numpy()
    tl64, dl64 = tl.double().numpy(), dl.double().numpy()
    for b in range(B):
        w = int(windows[b])
        r = oracle.accept_request(tl64[cu[b]:cu[b] + w], dl64[b * G1:b * G1 + w - 1],
                                  clamped[b, : w - 1], ua[b, : w - 1], ur[b])
        if any(m < 1e-6 for m in r["margins"]) or r["draw_margin"] < 1e-9:
            continue  # inside the flip band
        assert acc_h[b] == r["n"]
        n = r["n"]
        # the committed drafts are the tokens as given (the commit copies them)
        assert list(com_h[b, :n]) == list(tokens[b, :n]) and com_h[b, n] == r["committed"][n]


def test_schedule_bad_confidence():
    """A NaN and a 1.5 confidence: RVA_DEV_BAD_CONF, and the call still completes with
    windows inside [1, gamma]."""
    print("[status] schedule bad confidence", flush=True)
    B, gamma = 8, 5
    G = gamma - 1
    conf = np.full((B, G), 0.8, np.float32)
    conf[1, 2] = np.nan
    conf[4, 0] = 1.5
    alpha = np.zeros(B + 1, np.float32)
    theta = (np.float32(0.19) * np.arange(B * gamma + 1, dtype=np.float32)).astype(np.float32)
    conf_out = torch.empty((B, G), dtype=torch.float32, device=DEV)
    surv = torch.empty((B, G), dtype=torch.float32, device=DEV)
    windows = torch.empty(B, dtype=torch.int32, device=DEV)
    K = torch.empty(1, dtype=torch.int32, device=DEV)
    ratio = torch.empty(1, dtype=torch.float64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rva.schedule_windows(B, gamma, 0, None, 0, None, 0.0, d(conf), None, 20.0, d(alpha), d(theta),
                         conf_out, surv, windows, K, ratio, status)
    torch.cuda.synchronize()
    assert int(status.item()) & rva.DEV_BAD_CONF
    w = windows.cpu().numpy()
    assert np.all((w >= 1) & (w <= gamma))
