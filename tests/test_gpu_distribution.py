"""The acceptance kernels keep the target distribution, on the GPU, and handle masked logits.

"DSpark：投机解码与生产级 Serving 学习笔记", section 02: the acceptance rule compares the
target and draft distributions so that the committed tokens follow the target's
distribution exactly, and only a contiguous prefix of the drafts survives.  Two kinds of
tests run rva_accept_and_commit through the C ABI:

* test_target_distribution_kept: >= 10^6 seeded trials at V = 8 (float32 logits) and
  V = 1024 (bf16 logits), with drafts sampled from p_d.  Given that position k was reached
  (k drafts accepted), the committed token at position k must follow p_t of target row k
  whatever happened before: the accepted-draft part contributes min(p_d, p_t) and the
  residual draw max(0, p_t - p_d), which sum to p_t.  Checked per position by a chi-square
  test (bins with expected count < 5 pooled; p-value > 1e-3); the acceptance rate of the
  first draft must match the closed form sum_v min(p_t, p_d) = c* within 5 standard
  errors; no masked token may ever be committed.  The rows include masked (-inf) entries
  in both distributions, so the kernels' handling of zero probabilities is inside the
  check.  Inputs (logits, sampled drafts, uniforms) are drawn by torch with fixed seeds:
  they are the test's synthetic drafter, outside the path.
* test_accept_masked_parity: oracle parity on rows with -inf entries (random and a masked
  tail, so the last positive entry is not V - 1), drafted tokens with p_d(x) = 0 (reading:
  the ratio is +inf and the draft is accepted) and with p_t(x) = 0 (always rejected), and
  draws at u = 0 (first positive entry) and at the largest float32 below 1 (the draw lands
  on the last positive entry).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from ragged_verify_acceptance_amd import rva
from tests.reference import flip_band, record_flips

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rows(V, gamma, seed):
    """Target rows T_0..T_{gamma-1} and draft rows D_0..D_{gamma-2} (float32, with -inf)."""
    g = torch.Generator().manual_seed(seed)
    T = 2.0 * torch.randn((gamma, V), generator=g)
    D = T[: gamma - 1] + 0.8 * torch.randn((gamma - 1, V), generator=g)
    nmask = max(1, V // 8)
    for k in range(gamma):
        T[k, torch.randperm(V, generator=g)[:nmask]] = -float("inf")  # p_t = 0 entries
    for k in range(gamma - 1):
        D[k, torch.randperm(V, generator=g)[:nmask]] = -float("inf")  # p_d = 0 entries
    return T, D


@pytest.mark.parametrize("V,dtype", [(8, torch.float32), (1024, torch.bfloat16)], ids=["V8-f32", "V1024-bf16"])
def test_target_distribution_kept(V, dtype):
    print(f"[distribution] V={V} {dtype}", flush=True)
    gamma, B, calls = 4, 8192, 123  # 1,007,616 trials
    G1 = gamma - 1
    T, D = _rows(V, gamma, seed=V)
    T, D = T.to(dtype).float(), D.to(dtype).float()  # the values the kernel sees
    p_t = [oracle.softmax64(T[k].double().numpy()) for k in range(gamma)]
    p_d = [oracle.softmax64(D[k].double().numpy()) for k in range(G1)]
    tl = T.to(dtype).repeat(B, 1).contiguous().to(DEV)                     # [B*gamma, V]
    dl = D.to(dtype).unsqueeze(0).repeat(B, 1, 1).contiguous().to(DEV)     # [B, G1, V]
    cu = torch.arange(0, B * gamma + 1, gamma, dtype=torch.int32, device=DEV)
    pdist = torch.from_numpy(np.stack(p_d)).to(DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    com = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
    ctx = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, B * gamma), dtype=torch.uint8, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(12345 + V)
    hist = torch.zeros((gamma, V), dtype=torch.int64, device=DEV)
    first_accepts = 0
    for _ in range(calls):
        tokens = torch.stack([torch.multinomial(pdist[k], B, replacement=True, generator=g)
                              for k in range(G1)], dim=1).to(torch.int32).contiguous()
        u_acc = torch.rand((B, G1), generator=g, device=DEV)
        u_res = torch.rand(B, generator=g, device=DEV)
        rva.accept_and_commit(B, gamma, V, B * gamma, tl, dl, tokens, u_acc, u_res, cu, acc, com,
                              ctx, None, None, None, ws, status)
        n = acc.long()
        for k in range(gamma):
            sel = com[:, k][n >= k].long()
            hist[k] += torch.bincount(sel, minlength=V)
        first_accepts += int((n >= 1).sum().item())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hist = hist.cpu().numpy()
    trials = B * calls
    for k in range(gamma):
        h = hist[k]
        n_k = int(h.sum())
        assert np.all(h[p_t[k] == 0.0] == 0), f"position {k}: a masked token was committed"
        exp = p_t[k] * n_k
        big = exp >= 5.0
        obs_b = np.append(h[big], h[~big].sum())
        exp_b = np.append(exp[big], exp[~big].sum())
        keep = exp_b > 0
        chi2 = float(np.sum((obs_b[keep] - exp_b[keep]) ** 2 / exp_b[keep]))
        dof = int(keep.sum()) - 1
        p = float(stats.chi2.sf(chi2, dof))
        print(f"  position {k}: {n_k} tokens, chi2 {chi2:.1f} on {dof} dof, p = {p:.3g}")
        assert p > 1e-3, f"position {k}: committed tokens do not follow p_t (p = {p:.3g})"
    c_star = float(np.sum(np.minimum(p_t[0], p_d[0])))
    rate = first_accepts / trials
    se = np.sqrt(c_star * (1 - c_star) / trials)
    print(f"  first-draft acceptance {rate:.5f} vs c* {c_star:.5f} (se {se:.1e})")
    assert abs(rate - c_star) <= 5 * se


def test_accept_masked_parity():
    print("[accept-masked]", flush=True)
    rng = np.random.default_rng(77)
    B, gamma, V = 16, 6, 50_000
    G1 = gamma - 1
    windows = np.array([6, 6, 6, 6, 5, 4, 3, 2, 6, 6, 1, 6, 6, 6, 6, 6], np.int64)
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    max_rows = int(cu[-1]) + 1
    tl = (rng.standard_normal((max_rows, V)) * 2.0).astype(np.float32)
    dl = (rng.standard_normal((B * G1, V)) * 2.0).astype(np.float32)
    for b in range(B):  # close drafts: most drafts accepted, so later rows are reached
        for k in range(windows[b] - 1):
            dl[b * G1 + k] = tl[cu[b] + k] + 0.3 * rng.standard_normal(V).astype(np.float32)
    tl[rng.random(tl.shape) < 0.3] = -np.inf
    dl[rng.random(dl.shape) < 0.3] = -np.inf
    tl[:, V - 7000:] = -np.inf  # masked tail: the last positive target entry is below V - 7000
    tokens = rng.integers(0, V - 7000, size=(B, G1)).astype(np.int32)
    for b in range(B):
        for k in range(G1):
            if b % 4 == 1:  # p_d(x) = 0 (target finite): ratio +inf, accepted
                cand = np.flatnonzero(~np.isfinite(dl[b * G1 + k]) & np.isfinite(tl[cu[b] + min(k, windows[b] - 1)]))
                tokens[b, k] = int(cand[rng.integers(len(cand))])
            elif b % 4 == 2 and k == 0:  # p_d(x) = 0: accepted, so draft 2 is reached
                cand = np.flatnonzero(~np.isfinite(dl[b * G1 + k]) & np.isfinite(tl[cu[b] + min(k, windows[b] - 1)]))
                tokens[b, k] = int(cand[rng.integers(len(cand))])
            elif b % 4 == 2 and k == 1:  # p_t(x) = 0, p_d(x) > 0: ratio 0, rejected
                cand = np.flatnonzero(np.isfinite(dl[b * G1 + k]) & ~np.isfinite(tl[cu[b] + min(k, windows[b] - 1)]))
                tokens[b, k] = int(cand[rng.integers(len(cand))])
    ua = rng.random((B, G1)).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    ur[0::3] = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))  # last positive entry
    ur[1::5] = 0.0                                                        # first positive entry
    tl_t = torch.from_numpy(tl).to(torch.bfloat16)
    dl_t = torch.from_numpy(dl).to(torch.bfloat16)
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
    tl64, dl64 = tl_t.double().numpy(), dl_t.double().numpy()
    acc_h, com_h, ctx_h = acc.cpu().numpy(), com.cpu().numpy(), ctx.cpu().numpy()
    pt_h, pd_h, lab_h = pt.cpu().numpy(), pd.cpu().numpy(), lab.cpu().numpy()
    flips = 0
    saw_pd0_accept = saw_pt0_reject = saw_last = 0
    for b in range(B):
        w = int(windows[b])
        r = oracle.accept_request(tl64[cu[b]:cu[b] + w], dl64[b * G1:b * G1 + w - 1],
                                  tokens[b, : w - 1], ua[b, : w - 1], ur[b])
        same = acc_h[b] == r["n"] and list(com_h[b, : r["n"] + 1]) == list(r["committed"])
        if not same:
            assert flip_band(r), f"request {b}: {acc_h[b]} {com_h[b]} vs {r['n']} {r['committed']}"
            flips += 1
            continue
        assert np.all(com_h[b, r["n"] + 1:] == -1)
        assert ctx_h[b] == ctx0[b] + r["n"] + 1
        np.testing.assert_allclose(pt_h[b, : w - 1], r["pt_at"], atol=1e-5, rtol=0)
        np.testing.assert_allclose(pd_h[b, : w - 1], r["pd_at"], atol=1e-5, rtol=0)
        np.testing.assert_allclose(lab_h[b, : w - 1], r["labels"], atol=1e-5, rtol=0)
        y = int(com_h[b, r["n"]])
        row = tl64[cu[b] + r["n"]]
        assert np.isfinite(row[y]), f"request {b}: drew a masked token"
        saw_pd0_accept += sum(1 for k in range(r["n"]) if r["pd_at"][k] == 0.0)
        saw_pt0_reject += int(r["n"] < w - 1 and r["pt_at"][r["n"]] == 0.0)
        if ur[b] > 0.9999 and r["n"] == w - 1 and y == int(np.flatnonzero(np.isfinite(row))[-1]):
            saw_last += 1  # a bonus draw at u ~ 1 that lands on the last positive entry
    record_flips("accept-masked", B, flips)
    print(f"  p_d(x)=0 accepted: {saw_pd0_accept}, p_t(x)=0 rejected: {saw_pt0_reject}, "
          f"last-entry draws: {saw_last}, flips {flips}")
    assert saw_pd0_accept > 0 and saw_pt0_reject > 0 and saw_last > 0
    assert flips <= 1
