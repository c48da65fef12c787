"""Pins for the CPU oracle: values the pages print, closed forms, library special cases,
brute force on tiny inputs.  CPU only (no GPU needed).

Each test names what it would catch if the oracle had a plausible mistake.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.scheduling import step_cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- stage 1: survival


def test_survival_worked_table():
    """Printed survival table (DSpark study notes, section 07).  Catches a sum instead
    of a product, an off-by-one shift, or a product that restarts per position."""
    rows = _read_golden("survival_table.txt")
    c = np.array([[float(r[1]) for r in rows]], dtype=np.float32)
    printed = np.array([float(r[2]) for r in rows])
    a = oracle.survival(c)[0].astype(np.float64)
    assert np.all(np.abs(a - printed) <= 1e-3), (a, printed)
    # exact value of the fourth entry quoted in the fixture's header
    assert abs(a[3] - 0.5374656) < 1e-6


def test_survival_invariants():
    rng = np.random.default_rng(0)
    c = rng.uniform(0, 1, size=(50, 15)).astype(np.float32)
    a = oracle.survival(c)
    assert np.all(np.diff(a, axis=1) <= 0)  # non-increasing when c <= 1
    assert np.all(oracle.survival(np.ones((3, 7), np.float32)) == 1.0)
    assert np.array_equal(a[:, 0], c[:, 0])


# ---------------------------------------------------------------- stage 1: head + STS


def _hidden_for_logit(z, H=16):
    """hidden state whose head logit (w = e_0, b = 0) is exactly z."""
    h = np.zeros((1, len(z), H), dtype=np.float32)
    h[0, :, 0] = z
    w = np.zeros(H, dtype=np.float32)
    w[0] = 1.0
    return h, w


def test_confidence_head_closed_forms():
    """sigmoid(0) = 1/2, sigmoid(log 3) = 3/4, sigmoid(-log 3) = 1/4.  Catches a missing
    sign, a missing bias, or exp in place of the logistic function."""
    z = np.array([0.0, math.log(3.0), -math.log(3.0)], dtype=np.float32)
    h, w = _hidden_for_logit(z)
    c = oracle.confidence_from_head(h, w, 0.0)[0]
    assert abs(c[0] - 0.5) < 1e-7 and abs(c[1] - 0.75) < 1e-6 and abs(c[2] - 0.25) < 1e-6
    # the bias adds to the logit: z = 0 with b = log 3 gives 3/4
    c_b = oracle.confidence_from_head(h[:, :1], w, math.log(3.0))[0]
    assert abs(c_b[0] - 0.75) < 1e-6


def test_sts_identity_and_limits():
    """T = 1 is the identity; a huge temperature pushes every score to 1/2; the
    temperature divides the logit (T = 2 on logit 2 log 3 gives 3/4)."""
    rng = np.random.default_rng(1)
    h = rng.standard_normal((4, 5, 32)).astype(np.float32)
    w = (rng.standard_normal(32) / np.sqrt(32)).astype(np.float32)
    c0 = oracle.confidence_from_head(h, w, 0.3)
    c1 = oracle.confidence_from_head(h, w, 0.3, sts_T=np.ones(5, np.float32))
    assert np.array_equal(c0, c1)
    cinf = oracle.confidence_from_head(h, w, 0.3, sts_T=np.full(5, 1e30, np.float32))
    assert np.allclose(cinf, 0.5, atol=1e-7)
    z = np.array([2 * math.log(3.0)], dtype=np.float32)
    hz, wz = _hidden_for_logit(z)
    c2 = oracle.confidence_from_head(hz, wz, 0.0, sts_T=np.array([2.0], np.float32))[0, 0]
    assert abs(c2 - 0.75) < 1e-6


# ---------------------------------------------------------------- stage 1: scheduler


def _bruteforce_best(a, gamma, bias, alpha, theta):
    """Enumerate every window vector in [1, gamma]^B and return the best ratio and the
    set of vectors that reach it (an algorithm independent of the oracle's sort)."""
    B = a.shape[0]
    best, arg = -1.0, []
    for ws in itertools.product(range(1, gamma + 1), repeat=B):
        E = 0.0
        for b, wv in enumerate(ws):
            E += 1.0 + math.fsum(float(x) for x in a[b, : wv - 1])
        M = sum(ws)
        T = step_cost(bias, alpha, theta, B, M - B)
        r = E / T
        if r > best * (1 + 1e-12):
            best, arg = r, [ws]
        elif abs(r - best) <= 1e-12 * best:
            arg.append(ws)
    return best, arg


@pytest.mark.parametrize("seed", range(12))
def test_scheduler_matches_bruteforce(seed):
    """The sort-based argmax equals exhaustive search over all window vectors for
    B <= 4, gamma <= 5, on linear, convex and concave cost curves.  Catches a wrong
    tie rule, an objective without the +B bonus term, a theta indexed by K instead of
    bs + K, and a greedy stop that ends early."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 5))
    gamma = int(rng.integers(2, 6))
    c = rng.beta(4, 1.5, size=(B, gamma - 1)).astype(np.float32)
    a = oracle.survival(c)
    M = np.arange(B * gamma + 1, dtype=np.float64)
    kind = seed % 3
    slope = rng.uniform(0.05, 2.0)
    if kind == 0:
        theta = slope * M
    elif kind == 1:
        theta = slope * M + 0.02 * M ** 2
    else:
        theta = slope * 4 * np.sqrt(M)
    theta = theta.astype(np.float32)
    alpha = rng.uniform(0, 3, size=B + 1).astype(np.float32)
    bias = np.float32(rng.uniform(1, 20))
    res = oracle.schedule_windows(a, gamma, bias, alpha, theta)
    best, arg = _bruteforce_best(a, gamma, bias, alpha, theta)
    assert abs(res["ratio"] - best) <= 1e-12 * best
    assert tuple(int(x) for x in res["windows"]) in arg
    # the reported K is the number of verified drafts
    assert res["K"] == int(res["windows"].sum()) - B


def test_scheduler_limits():
    """Free verification (theta = 0) keeps every full window; prohibitively expensive
    verification trims every window to the anchor alone; static mode is gamma."""
    rng = np.random.default_rng(7)
    B, gamma = 5, 7
    a = oracle.survival(rng.uniform(0.2, 0.99, size=(B, gamma - 1)).astype(np.float32))
    zero = np.zeros(B * gamma + 1, np.float32)
    r0 = oracle.schedule_windows(a, gamma, 20.0, zero[: B + 1], zero)
    assert np.all(r0["windows"] == gamma)
    huge = (1e6 * np.arange(B * gamma + 1)).astype(np.float32)
    r1 = oracle.schedule_windows(a, gamma, 1.0, zero[: B + 1], huge)
    assert np.all(r1["windows"] == 1)
    rs = oracle.schedule_windows(a, gamma, 1.0, zero[: B + 1], huge, static=True)
    assert np.all(rs["windows"] == gamma) and rs["K"] == B * (gamma - 1)


def test_scheduler_batch_effect_derived():
    """Derived (not printed on the pages): every request carries the worked survival
    table and T = 20 ms + 0.19 ms/token (SGLang article, "Background" figure).  A batch
    of one verifies the full block (the pages say trimming saves little at batch 1);
    windows shrink as the batch grows (6 / 5 / 4 / 3 at B = 1 / 16 / 64 / 256)."""
    rows = _read_golden("survival_table.txt")
    cost = {r[0]: float(r[1]) for r in _read_golden("step_cost.txt")}
    c = np.array([float(r[1]) for r in rows], dtype=np.float32)
    for B, mean_w in [(1, 6.0), (16, 5.0), (64, 4.0), (256, 3.0)]:
        a = oracle.survival(np.tile(c, (B, 1)))
        theta = (np.float32(cost["theta_ms_per_token"]) * np.arange(B * 6 + 1)).astype(np.float32)
        alpha = np.full(B + 1, cost["alpha_ms"], np.float32)
        r = oracle.schedule_windows(a, 6, cost["bias_ms"], alpha, theta)
        assert r["windows"].mean() == mean_w


def test_scheduler_tie_rule():
    """Equal survivals across requests are taken in request order; a plateau of zero
    survivals under a constant cost ties, and the smallest K wins."""
    a = np.array([[0.9, 0.0], [0.9, 0.0]], dtype=np.float32)
    zero = np.zeros(7, np.float32)
    r = oracle.schedule_windows(a, 3, 10.0, zero[:3], zero)
    assert list(r["windows"]) == [2, 2] and r["K"] == 2
    # a cost that makes exactly one extra draft worthwhile goes to request 0
    theta = np.array([0, 0, 0, 0.5, 100, 100, 100], np.float32)
    r = oracle.schedule_windows(a, 3, 10.0, zero[:3], theta)
    assert list(r["windows"]) == [2, 1]


# ---------------------------------------------------------------- stage 2: packing


def test_tier_example():
    """Printed packing example (SGLang article, ragged verify figure)."""
    g = {r[0]: [int(x) for x in r[1:]] for r in _read_golden("tier_example.txt")}
    res = oracle.pack_ragged(g["windows"], [100, 200, 300], g["tiers"])
    assert list(res["cu_seqlens"]) == g["cu_seqlens"]
    assert res["M"] == g["total"][0] and res["tier"] == g["tier"][0]
    # rows 10, 11 are padding; rows of request 1 sit at positions 200..202
    assert list(res["row_req"][:12]) == [0] * 5 + [1] * 3 + [2] * 2 + [-1, -1]
    assert list(res["row_pos"][5:8]) == [200, 201, 202]


def test_pack_rows_and_padding():
    rng = np.random.default_rng(3)
    B, gamma, H = 9, 6, 5
    windows = rng.integers(1, gamma + 1, size=B)
    src = rng.standard_normal((B, gamma, H)).astype(np.float32)
    tiers = [8, 16, 32, 64]
    res = oracle.pack_ragged(windows, np.arange(B) * 10, tiers, src, max_rows=64)
    M = int(windows.sum())
    assert res["M"] == M and res["tier"] == min(t for t in tiers if t >= M)
    r = 0
    for b in range(B):
        for i in range(int(windows[b])):
            assert np.array_equal(res["dst"][r], src[b, i])
            r += 1
    assert np.all(res["dst"][M:] == 0)
    with pytest.raises(ValueError):
        oracle.pack_ragged([6] * B, [0] * B, [8, 16])


# ---------------------------------------------------------------- stage 3: attention


def _paged_case(rng, B=3, Hq=4, Hkv=2, D=16, page=4, lens=(0, 5, 9), windows=(3, 2, 4)):
    """Tiny paged case with a scrambled page table.  Returns a dict of oracle inputs."""
    need = [(L + w + page - 1) // page for L, w in zip(lens, windows)]
    max_pages = max(need)
    P = sum(need) + 3
    perm = rng.permutation(P)
    bt = np.zeros((B, max_pages), np.int32)
    k = 0
    for b in range(B):
        for j in range(need[b]):
            bt[b, j] = perm[k]
            k += 1
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    R = int(cu[-1]) + 2
    return dict(
        q=rng.standard_normal((R, Hq, D)),
        k_new=rng.standard_normal((R, Hkv, D)),
        v_new=rng.standard_normal((R, Hkv, D)),
        k_cache=rng.standard_normal((P, Hkv, page, D)),
        v_cache=rng.standard_normal((P, Hkv, page // oracle.attention.v_block(page), D,
                                     oracle.attention.v_block(page))),
        block_table=bt,
        context_lens=np.array(lens, np.int32),
        cu_seqlens=cu,
        tier=R,
        softmax_scale=np.float32(1 / math.sqrt(D)),
    )


def _logical_kv(case, b, g):
    """Context K/V of request b, kv head g, in position order (test-side gather)."""
    L = int(case["context_lens"][b])
    page = case["k_cache"].shape[2]
    D = case["k_cache"].shape[3]
    K = np.zeros((L, D))
    V = np.zeros((L, D))
    for p in range(L):
        K[p] = case["k_cache"][case["block_table"][b, p // page], g, p % page]
        VB = case["v_cache"].shape[4]
        s = p % page
        V[p] = case["v_cache"][case["block_table"][b, p // page], g, s // VB, :, s % VB]
    return K, V


@pytest.mark.parametrize("page,lens", [(4, (0, 5, 9)), (64, (0, 70, 131))])
def test_attention_against_torch_sdpa(page, lens):
    """Library special case: per request, masked scaled-dot-product attention from
    torch (float64, CPU) over [context ; window] with a causal window mask.  Catches a
    wrong scale, a missing causal mask, a mask that lets a row see later window rows,
    a wrong GQA group mapping, and a wrong slot -> V column-block mapping (page 64
    holds two 32-slot blocks)."""
    rng = np.random.default_rng(11)
    case = _paged_case(rng, page=page, lens=lens)
    out, _, _ = oracle.verify_attention(**case)
    Hq, Hkv = case["q"].shape[1], case["k_new"].shape[1]
    for b in range(3):
        L = int(case["context_lens"][b])
        r0, r1 = int(case["cu_seqlens"][b]), int(case["cu_seqlens"][b + 1])
        w = r1 - r0
        mask = np.zeros((w, L + w), bool)
        for i in range(w):
            mask[i, : L + i + 1] = True
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Kc, Vc = _logical_kv(case, b, g)
            K = np.concatenate([Kc, case["k_new"][r0:r1, g]])
            V = np.concatenate([Vc, case["v_new"][r0:r1, g]])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(case["q"][r0:r1, h][None]), torch.from_numpy(K[None]),
                torch.from_numpy(V[None]), attn_mask=torch.from_numpy(mask[None]),
                scale=float(case["softmax_scale"]))[0].numpy()
            assert np.allclose(out[r0:r1, h], ref, rtol=1e-10, atol=1e-12)
    assert np.all(out[int(case["cu_seqlens"][-1]):] == 0)


@pytest.mark.parametrize("page", [32, 64, 16])
def test_attention_cache_layout_from_logical(page):
    """The cache layout pinned from the other side: logical context K/V [L, D] per (request,
    kv head) are written into pages by whole-page reshapes (K page = the [page, D] block of
    its positions; V page = that block cut into column blocks of VB slots and transposed
    to [page/VB, D, VB], as the header states the layout), never by the oracle's element
    index.  The oracle's output must equal torch SDPA on the logical K/V, and the window
    it appends must read back, by the inverse reshape, at positions L .. L+w-1."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, D = 3, 4, 2, 8
    lens, windows = (0, 40, 77), (2, 3, 4)
    VB = oracle.attention.v_block(page)
    need = [(L + w + page - 1) // page for L, w in zip(lens, windows)]
    P = sum(need) + 2
    perm = rng.permutation(P)
    bt = np.zeros((B, max(need)), np.int32)
    k = 0
    for b in range(B):
        for j in range(need[b]):
            bt[b, j] = perm[k]
            k += 1
    k_cache = rng.standard_normal((P, Hkv, page, D))   # untouched slots keep noise
    v_cache = rng.standard_normal((P, Hkv, page // VB, D, VB))
    logical = {}
    for b in range(B):
        for g in range(Hkv):
            Kl = rng.standard_normal((lens[b], D))
            Vl = rng.standard_normal((lens[b], D))
            logical[b, g] = (Kl, Vl)
            for j in range((lens[b] + page - 1) // page):
                n = min(page, lens[b] - j * page)
                kb = k_cache[bt[b, j], g].copy()
                kb[:n] = Kl[j * page: j * page + n]
                k_cache[bt[b, j], g] = kb
                vb = v_cache[bt[b, j], g].transpose(0, 2, 1).reshape(page, D).copy()  # [slot, d]
                vb[:n] = Vl[j * page: j * page + n]
                v_cache[bt[b, j], g] = vb.reshape(page // VB, VB, D).transpose(0, 2, 1)
    cu = np.concatenate([[0], np.cumsum(windows)]).astype(np.int32)
    R = int(cu[-1])
    q = rng.standard_normal((R, Hq, D))
    k_new = rng.standard_normal((R, Hkv, D))
    v_new = rng.standard_normal((R, Hkv, D))
    scale = np.float32(1 / math.sqrt(D))
    out, kc, vc = oracle.verify_attention(q, k_new, v_new, k_cache.copy(), v_cache.copy(), bt,
                                          np.array(lens, np.int32), cu, R, scale)
    G = Hq // Hkv
    for b in range(B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        w = r1 - r0
        for h in range(Hq):
            g = h // G
            Kl, Vl = logical[b, g]
            K = np.concatenate([Kl, k_new[r0:r1, g]])
            V = np.concatenate([Vl, v_new[r0:r1, g]])
            mask = np.ones((w, lens[b] + w), bool)
            for i in range(w):
                mask[i, lens[b] + i + 1:] = False
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[r0:r1, h][None]), torch.from_numpy(K[None]), torch.from_numpy(V[None]),
                attn_mask=torch.from_numpy(mask[None]), scale=float(scale))[0].numpy()
            assert np.allclose(out[r0:r1, h], ref, rtol=1e-10, atol=1e-12), (page, b, h)
        # the appended window, read back page by page with the inverse reshape
        for g in range(Hkv):
            for i in range(w):
                p = lens[b] + i
                pg, s = bt[b, p // page], p % page
                vpage = vc[pg, g].transpose(0, 2, 1).reshape(page, D)
                assert np.array_equal(kc[pg, g, s], k_new[r0 + i, g])
                assert np.array_equal(vpage[s], v_new[r0 + i, g])


def test_attention_special_cases():
    """Single visible key -> its value; zero query -> mean of the visible values;
    GQA equals MHA with every kv head repeated; physical page order is irrelevant."""
    rng = np.random.default_rng(12)
    case = _paged_case(rng)
    # request 0 has no context: its first row sees only itself
    out, kc, vc = oracle.verify_attention(**case)
    for h in range(4):
        assert np.allclose(out[0, h], case["v_new"][0, h // 2])
    # zero query: uniform weights over the visible keys
    zc = dict(case, q=np.zeros_like(case["q"]))
    outz, _, _ = oracle.verify_attention(**zc)
    b, i = 1, 1
    r = int(case["cu_seqlens"][b]) + i
    for h in range(4):
        g = h // 2
        Kc, Vc = _logical_kv(case, b, g)
        vis = np.concatenate([Vc, case["v_new"][int(case["cu_seqlens"][b]): r + 1, g]])
        assert np.allclose(outz[r, h], vis.mean(axis=0))
    # GQA vs MHA with repeated kv heads
    mha = dict(case, k_new=np.repeat(case["k_new"], 2, axis=1), v_new=np.repeat(case["v_new"], 2, axis=1),
               k_cache=np.repeat(case["k_cache"], 2, axis=1), v_cache=np.repeat(case["v_cache"], 2, axis=1))
    outm, _, _ = oracle.verify_attention(**mha)
    assert np.allclose(outm, out, rtol=1e-12, atol=1e-14)
    # relabel the physical pages
    P = case["k_cache"].shape[0]
    perm = rng.permutation(P)
    inv = np.argsort(perm)
    rel = dict(case, k_cache=case["k_cache"][inv], v_cache=case["v_cache"][inv],
               block_table=perm[case["block_table"]].astype(np.int32))
    outp, _, _ = oracle.verify_attention(**rel)
    assert np.allclose(outp, out, rtol=1e-12, atol=1e-14)


def test_attention_causal_and_append():
    """Changing window row j's K/V leaves rows i < j unchanged; after the call the cache
    holds the window's K/V at positions L .. L+w-1 and nothing else changed."""
    rng = np.random.default_rng(13)
    case = _paged_case(rng)
    out, kc, vc = oracle.verify_attention(**case)
    b, j = 2, 2
    r0 = int(case["cu_seqlens"][b])
    pert = dict(case, k_new=case["k_new"].copy(), v_new=case["v_new"].copy())
    pert["k_new"][r0 + j] += 5.0
    pert["v_new"][r0 + j] -= 3.0
    outp, _, _ = oracle.verify_attention(**pert)
    assert np.array_equal(outp[r0:r0 + j], out[r0:r0 + j])
    assert not np.allclose(outp[r0 + j], out[r0 + j])
    page = case["k_cache"].shape[2]
    touched = set()
    for bb in range(3):
        L = int(case["context_lens"][bb])
        rr = int(case["cu_seqlens"][bb])
        for i in range(int(case["cu_seqlens"][bb + 1]) - rr):
            p = L + i
            pg, s = case["block_table"][bb, p // page], p % page
            assert np.array_equal(kc[pg, :, s, :], case["k_new"][rr + i])
            VB = vc.shape[4]
            assert np.array_equal(vc[pg, :, s // VB, :, s % VB], case["v_new"][rr + i])
            touched.add((int(pg), s))
    for pg in range(case["k_cache"].shape[0]):
        for s in range(page):
            if (pg, s) not in touched:
                assert np.array_equal(kc[pg, :, s], case["k_cache"][pg, :, s])


# ---------------------------------------------------------------- stages 4-5


def test_inverse_cdf_small():
    q = [0.2, 0.3, 0.5]
    assert oracle.inverse_cdf(q, 0.0)[0] == 0
    assert oracle.inverse_cdf(q, 0.1)[0] == 0
    assert oracle.inverse_cdf(q, 0.2)[0] == 1  # C_0 = 0.2 is not > 0.2
    assert oracle.inverse_cdf(q, 0.49)[0] == 1
    assert oracle.inverse_cdf(q, 0.5)[0] == 2
    assert oracle.inverse_cdf(q, 0.999)[0] == 2
    assert oracle.inverse_cdf([0, 0, 4.0, 0], 0.7)[0] == 2  # one-hot
    assert oracle.inverse_cdf([2.0, 2.0], 0.5)[0] == 1  # unnormalised weights


def test_tv_label_closed_forms():
    """Hand example p_d = (0.7, 0.3), p_t = (0.4, 0.6): TV = 0.3, label 0.7; the label
    equals sum(min(p_d, p_t)), is symmetric, 1 on equal rows, in [0, 1]."""
    assert abs(oracle.acceptance.tv_label([0.7, 0.3], [0.4, 0.6]) - 0.7) < 1e-15
    rng = np.random.default_rng(5)
    for _ in range(20):
        a = oracle.softmax64(rng.normal(0, 2, 50))
        b = oracle.softmax64(rng.normal(0, 2, 50))
        lab = oracle.acceptance.tv_label(a, b)
        assert abs(lab - np.minimum(a, b).sum()) < 1e-14
        assert abs(lab - oracle.acceptance.tv_label(b, a)) < 1e-15
        assert 0 <= lab <= 1
        # the residual mass max(0, p_t - p_d) is 1 - label
        assert abs(np.maximum(0, b - a).sum() - (1 - lab)) < 1e-14
        assert abs(oracle.acceptance.tv_label(a, a) - 1.0) < 1e-15


def test_softmax_library_special_case():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 2, 1000)
    ref = torch.softmax(torch.from_numpy(x), dim=0).numpy()
    assert np.allclose(oracle.softmax64(x), ref, rtol=1e-13, atol=1e-300)


def test_prefix_only_acceptance():
    """Reject at draft 2 while draft 3 would be accepted on its own: only draft 1 is
    committed, followed by the residual draw (DSpark study notes, section 02)."""
    V = 6
    t = np.log(np.array([[0.5, 0.1, 0.1, 0.1, 0.1, 0.1],
                         [0.05, 0.05, 0.3, 0.3, 0.2, 0.1],
                         [0.1, 0.1, 0.1, 0.1, 0.1, 0.5],
                         [0.2, 0.2, 0.2, 0.2, 0.1, 0.1]]))
    d = np.log(np.array([[0.5, 0.1, 0.1, 0.1, 0.1, 0.1],    # draft 1 == target row 0
                         [0.05, 0.8, 0.05, 0.05, 0.025, 0.025],  # draft 2 puts 0.8 on token 1
                         [0.1, 0.1, 0.1, 0.1, 0.1, 0.5]]))  # draft 3 == target row 2
    tokens = [0, 1, 5]
    u = [0.3, 0.5, 0.01]  # draft 2: r = 0.05/0.8 = 0.0625 < 0.5 -> reject
    res = oracle.accept_request(t, d, tokens, u, 0.0)
    assert res["n"] == 1 and len(res["committed"]) == 2 and res["committed"][0] == 0
    # residual max(0, p_t[1] - p_d[2]) is zero on token 1 and 0; u' = 0 -> first token
    # with positive residual mass
    resid = np.maximum(0, np.exp(t[1]) - np.exp(d[1]))
    assert resid[1] == 0 and res["committed"][1] == int(np.nonzero(resid > 0)[0][0])
    assert len(res["margins"]) == 2  # draft 3 is never evaluated


def test_equal_distributions_accept_all():
    rng = np.random.default_rng(8)
    t = rng.normal(0, 2, size=(5, 30))
    d = t[:4].copy()
    tokens = rng.integers(0, 30, 4)
    res = oracle.accept_request(t, d, tokens, rng.uniform(0, 1, 4), 0.37)
    assert res["n"] == 4
    assert res["committed"][-1] == oracle.inverse_cdf(oracle.softmax64(t[4]), 0.37)[0]
    assert np.allclose(res["labels"], 1.0)


def _mc_accept(t, d, trials, seed):
    """Monte Carlo of the acceptance rule with draft tokens drawn from p_d."""
    rng = np.random.default_rng(seed)
    pd = [oracle.softmax64(r) for r in d]
    w = len(t)
    out = np.zeros((trials, w), np.int64) - 1
    ns = np.zeros(trials, np.int64)
    for n in range(trials):
        toks = [rng.choice(len(p), p=p) for p in pd]
        res = oracle.accept_request(t, d, toks, rng.uniform(size=w - 1).astype(np.float32),
                                    np.float32(rng.uniform()))
        out[n, : len(res["committed"])] = res["committed"]
        ns[n] = res["n"]
    return out, ns


def _chi2_pvalue(counts, probs):
    from scipy.stats import chisquare

    n = counts.sum()
    exp = probs * n
    keep = exp > 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return chisquare(obs, ex * obs.sum() / ex.sum()).pvalue


def test_target_distribution_preserved():
    """The committed token at each position follows the target row that verifies it
    (DSpark study notes, section 02; SGLang article, "Background").  V = 8, window 3,
    draft rows far from the target rows.  Catches a ratio inverted, a residual with the
    wrong sign, a bonus taken from the wrong row, and drafts verified by the wrong row."""
    rng = np.random.default_rng(21)
    V, w = 8, 3
    t = rng.normal(0, 1.5, size=(w, V))
    d = rng.normal(0, 1.5, size=(w - 1, V))
    trials = 60000
    out, ns = _mc_accept(t, d, trials, seed=22)
    pt = [oracle.softmax64(r) for r in t]
    # position 0 always holds a committed token distributed as p_t[0]
    c0 = np.bincount(out[:, 0], minlength=V)
    assert _chi2_pvalue(c0, pt[0]) > 1e-3
    # given draft 1 was accepted, position 1 is distributed as p_t[1]
    sel = out[ns >= 1, 1]
    assert _chi2_pvalue(np.bincount(sel, minlength=V), pt[1]) > 1e-3
    sel = out[ns >= 2, 2]
    assert _chi2_pvalue(np.bincount(sel, minlength=V), pt[2]) > 1e-3


def test_acceptance_rate_equals_label():
    """Per-position acceptance probability equals the TV label sum(min(p_d, p_t)), and the
    expected accepted length is sum_j prod_{i<=j} c*_i for independent rows."""
    rng = np.random.default_rng(31)
    V, w = 8, 4
    t = rng.normal(0, 1.0, size=(w, V))
    d = t[: w - 1] + rng.normal(0, 0.7, size=(w - 1, V))
    trials = 40000
    out, ns = _mc_accept(t, d, trials, seed=32)
    cstar = [oracle.acceptance.tv_label(oracle.softmax64(d[k]), oracle.softmax64(t[k])) for k in range(w - 1)]
    p1 = (ns >= 1).mean()
    assert abs(p1 - cstar[0]) < 4 * math.sqrt(cstar[0] * (1 - cstar[0]) / trials)
    expect = sum(np.prod(cstar[: j + 1]) for j in range(w - 1))
    sd = ns.std() / math.sqrt(trials)
    assert abs(ns.mean() - expect) < 4 * sd


def test_batch_driver_layout():
    """accept_and_commit reads draft k against packed target row cu[b] + k - 1 and
    advances context_lens by n + 1."""
    rng = np.random.default_rng(41)
    B, gamma, V = 3, 4, 12
    windows = np.array([4, 1, 2])
    cu = np.concatenate([[0], np.cumsum(windows)])
    tl = rng.normal(0, 2, size=(int(cu[-1]) + 1, V))
    dl = rng.normal(0, 2, size=(B, gamma - 1, V))
    toks = rng.integers(0, V, size=(B, gamma - 1))
    ua = rng.uniform(size=(B, gamma - 1)).astype(np.float32)
    ur = rng.uniform(size=B).astype(np.float32)
    res = oracle.accept_and_commit(tl, dl, toks, ua, ur, windows, cu, [10, 20, 30])
    for b in range(B):
        w = int(windows[b])
        one = oracle.accept_request(tl[cu[b]:cu[b] + w], dl[b, : w - 1], toks[b, : w - 1], ua[b, : w - 1], ur[b])
        n = one["n"]
        assert res["accept_len"][b] == n
        assert list(res["committed"][b, : n + 1]) == one["committed"]
        assert np.all(res["committed"][b, n + 1:] == -1)
        assert res["context_lens"][b] == [10, 20, 30][b] + n + 1
        assert np.all(np.isnan(res["labels"][b, w - 1:]))
    # window 1: no drafts verified, the bonus comes from the request's only row
    assert res["accept_len"][1] == 0
    assert res["committed"][1, 0] == oracle.inverse_cdf(oracle.softmax64(tl[cu[1]]), ur[1])[0]
    lab = oracle.confidence_labels(tl, dl, windows, cu)
    assert np.allclose(lab, res["labels"], equal_nan=True)


# ---------------------------------------------------------------- cap-accept verify mode


def test_cap_accept_commits_what_compact_commits():
    """Cap-accept ([SGL] "Confidence scheduler 与 verify 模式"; [CSDN] section 5) verifies the
    whole block but commits only inside the window: its commit must equal compact mode's
    commit for that window, and its ceiling must equal the whole block's (static mode's)
    acceptance.  Checked over many seeded cases, with drafts close to the target (long
    acceptances, so the cap binds) and far from it (early rejections)."""
    rng = np.random.default_rng(21)
    checked_binding = checked_free = 0
    for case in range(300):
        V, w = 12, int(rng.integers(1, 8))
        t = rng.standard_normal((w, V)) * 1.5
        noise = 0.05 if case % 2 == 0 else 1.5
        d = t[: w - 1] + rng.standard_normal((w - 1, V)) * noise
        tokens = np.array([int(np.argmax(d[k] + rng.gumbel(size=V))) for k in range(w - 1)], np.int64)
        ua = rng.random(w - 1).astype(np.float32)
        ur = np.float32(rng.random())
        full = oracle.accept_request(t, d, tokens, ua, ur)
        for cap in range(1, w + 1):
            capped = oracle.accept_request_capped(t, d, tokens, ua, ur, cap)
            compact = oracle.accept_request(t[:cap], d[: cap - 1], tokens[: cap - 1], ua[: cap - 1], ur)
            assert capped["n"] == compact["n"]
            assert capped["committed"] == compact["committed"]
            assert capped["n_full"] == full["n"]
            assert capped["n"] <= capped["n_full"]
            if capped["n_full"] > capped["n"]:
                checked_binding += 1
            else:
                checked_free += 1
            if cap == w:  # no cap: the whole-block result
                assert capped["committed"] == full["committed"]
            np.testing.assert_allclose(capped["labels"], full["labels"], rtol=0, atol=0)
    assert checked_binding > 50 and checked_free > 50
