"""Oracle-side expected values for a workload (test infrastructure).

Builds the oracle's inputs from the same seeded generator the device harness uses and runs
the oracle on all requests or on a sample of them.  Never touches the GPU path.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import Inputs


def oracle_conf(inp: Inputs) -> np.ndarray:
    wl = inp.wl
    if wl.conf_from_head:
        return oracle.confidence_from_head(inp.hidden().float().numpy(), inp.head_w, inp.head_b)
    return inp.conf()


def oracle_schedule(inp: Inputs, static=False):
    c = oracle_conf(inp)
    a = oracle.survival(c)
    bias, alpha, theta = inp.cost_tables()
    r = oracle.schedule_windows(a, inp.wl.gamma, bias, alpha, theta, static=static)
    r["c"] = c
    r["a"] = a
    return r


def sub_pool(inp: Inputs, reqs):
    """Compact page pools holding only the context pages of `reqs` (oracle layout), with
    the block table of those requests renumbered into them."""
    wl = inp.wl
    pages = []
    for b in reqs:
        pages.extend(int(p) for p in inp.block_table[b, : int(inp.pages_per_req[b])])
    local = {p: i for i, p in enumerate(sorted(pages))}
    P = len(local)
    k_pool = np.full((P, wl.Hkv, wl.page, wl.D), np.nan)
    VB = oracle.attention.v_block(wl.page)
    v_pool = np.full((P, wl.Hkv, wl.page // VB, wl.D, VB), np.nan)
    bt = np.zeros((len(reqs), inp.max_pages), np.int32)
    for j, b in enumerate(reqs):
        K, V = inp.request_context_kv(b)
        K = K.double().numpy()
        V = V.double().numpy()
        L = int(inp.context_lens[b])
        for pj in range(int(inp.pages_per_req[b])):
            lp = local[int(inp.block_table[b, pj])]
            bt[j, pj] = lp
            lo, hi = pj * wl.page, min(L, (pj + 1) * wl.page)
            if hi > lo:
                k_pool[lp, :, : hi - lo, :] = K[lo:hi].transpose(1, 0, 2)
                for s0 in range(lo, hi):
                    v_pool[lp, :, (s0 - lo) // VB, :, (s0 - lo) % VB] = V[s0]
    return k_pool, v_pool, bt, local


def oracle_attention(inp: Inputs, windows, reqs):
    """Oracle attention for the requests `reqs` (a sub-batch).  Returns
    {b: out rows [w_b, Hq, D]} and {b: (K_window [w, Hkv, D], V_window)} (the appended KV)."""
    wl = inp.wl
    k_pool, v_pool, bt, _ = sub_pool(inp, reqs)
    ws = [int(windows[b]) for b in reqs]
    cu = np.concatenate([[0], np.cumsum(ws)]).astype(np.int32)
    R = int(cu[-1])
    q = np.zeros((R, wl.Hq, wl.D))
    kn = np.zeros((R, wl.Hkv, wl.D))
    vn = np.zeros((R, wl.Hkv, wl.D))
    for j, b in enumerate(reqs):
        qb, kb, vb = inp.request_qkv(b)
        q[cu[j]:cu[j + 1]] = qb[: ws[j]].double().numpy()
        kn[cu[j]:cu[j + 1]] = kb[: ws[j]].double().numpy()
        vn[cu[j]:cu[j + 1]] = vb[: ws[j]].double().numpy()
    out, kc, vc = oracle.verify_attention(q, kn, vn, k_pool, v_pool, bt,
                                          inp.context_lens[list(reqs)], cu, R,
                                          np.float32(1.0 / np.sqrt(wl.D)))
    res = {b: out[cu[j]:cu[j + 1]] for j, b in enumerate(reqs)}
    app = {b: (kn[cu[j]:cu[j + 1]], vn[cu[j]:cu[j + 1]]) for j, b in enumerate(reqs)}
    return res, app, (kc, vc, bt)


def oracle_accept(inp: Inputs, windows, reqs):
    """Per-request acceptance results for `reqs`: {b: accept_request dict}."""
    ua, ur = inp.uniforms()
    res = {}
    for b in reqs:
        w = int(windows[b])
        tl, dl, toks = inp.request_logits(b)
        r = oracle.accept_request(tl[:w].double().numpy(), dl[: w - 1].double().numpy(),
                                  toks[: w - 1], ua[b, : w - 1], ur[b])
        res[b] = r
    return res


def oracle_accept_capped(inp: Inputs, caps, reqs):
    """Cap-accept results for `reqs`: the whole block verified, commit capped at caps[b]."""
    ua, ur = inp.uniforms()
    res = {}
    w = inp.wl.gamma
    for b in reqs:
        tl, dl, toks = inp.request_logits(b)
        res[b] = oracle.accept_request_capped(tl[:w].double().numpy(), dl[: w - 1].double().numpy(),
                                              toks[: w - 1], ua[b, : w - 1], ur[b], int(caps[b]))
    return res


def attn_rel_err(out, ref):
    """max over (row, head) vectors of max|o - r| / max|r|."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / den))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().float().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()
