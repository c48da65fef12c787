"""Oracle for stages 4 and 5: speculative-sampling acceptance, commit, TV labels.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product path.

Row alignment used throughout: draft k (k = 1 .. w-1, token ``draft_tokens[b, k-1]``,
logits ``draft_logits[b, k-1]``) is verified by packed target row ``cu[b] + k - 1``
(the target's distribution for the position that draft k fills, conditioned on the
anchor and drafts 1 .. k-1); the bonus token comes from target row ``cu[b] + w - 1``.
"""

from __future__ import annotations

import numpy as np


def softmax64(logits):
    """Softmax of one logit row in float64 (temperature 1)."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def inverse_cdf(q, u):
    """Draw from the unnormalised weights ``q`` with one uniform ``u`` in [0, 1).

    Inverse CDF in ascending token order: ``S = sum(q)`` and the cumulative sums ``C_v``
    are formed left to right in float64; the result is the smallest v with
    ``C_v > u * S``.  Returns (v, margin) where margin is the distance of ``u * S`` to the
    nearest bin edge of the chosen bin, relative to S (used to count boundary flips).
    """
    q = np.asarray(q, dtype=np.float64)
    C = np.cumsum(q)  # sequential, index order
    S = float(C[-1])
    t = float(u) * S
    v = int(np.searchsorted(C, t, side="right"))
    v = min(v, len(q) - 1)
    lo = float(C[v - 1]) if v > 0 else 0.0
    hi = float(C[v])
    margin = min(abs(t - lo), abs(hi - t)) / S if S > 0 else 0.0
    return v, margin


def accept_request(target_rows, draft_rows, tokens, u_accept, u_resample):
    """Acceptance and commit for one request with window ``w = len(target_rows)``.

    [NOTES] section 02: acceptance compares the target and draft distributions in a way
    that keeps the target's output distribution, and it is prefix-only: after the first
    rejection nothing later is kept.  [SGL] "Background": every verify forward also yields
    one target token.  The rule used is the standard speculative-sampling rule at
    temperature 1:

    * for k = 1 .. w-1 with x = draft token k: ``r = p_t[k-1](x) / p_d[k](x)``
      (``+inf`` when ``p_d(x) = 0``); accept iff ``u_k < min(1, r)``;
    * on the first rejection at k: draw y from ``max(0, p_t[k-1] - p_d[k])`` (renormalised;
      if that residual is identically zero, from ``p_t[k-1]``) and stop;
    * if every draft is accepted: draw the bonus y from ``p_t[w-1]``;
    * commit ``x_1 .. x_n, y`` (n accepted drafts).

    Draws use ``inverse_cdf`` with the request's single uniform ``u_resample``.
    Returns dict(n, committed list, margins (|u - r| per evaluated k), draw_margin,
    labels [w-1], pt_at [w-1], pd_at [w-1]).
    """
    w = len(target_rows)
    p_t = [softmax64(r) for r in target_rows]
    p_d = [softmax64(r) for r in draft_rows]
    pt_at = [float(p_t[k - 1][int(tokens[k - 1])]) for k in range(1, w)]
    pd_at = [float(p_d[k - 1][int(tokens[k - 1])]) for k in range(1, w)]
    labels = [tv_label(p_d[k - 1], p_t[k - 1]) for k in range(1, w)]
    n = 0
    margins = []
    residual = None
    for k in range(1, w):
        pt, pd = pt_at[k - 1], pd_at[k - 1]
        r = np.inf if pd == 0.0 else pt / pd
        u = float(np.float32(u_accept[k - 1]))
        margins.append(abs(u - r))
        if u < min(1.0, r):
            n += 1
            continue
        residual = np.maximum(0.0, p_t[k - 1] - p_d[k - 1])
        if not np.sum(residual) > 0.0:
            residual = p_t[k - 1]
        break
    if residual is None:
        residual = p_t[w - 1]
    y, draw_margin = inverse_cdf(residual, float(np.float32(u_resample)))
    committed = [int(tokens[i]) for i in range(n)] + [y]
    return {"n": n, "committed": committed, "margins": margins, "draw_margin": draw_margin,
            "labels": labels, "pt_at": pt_at, "pd_at": pd_at}


def tv_label(p_d, p_t):
    """TV-distance confidence label ``c* = 1 - 0.5 * ||p_d - p_t||_1``.

    [NOTES] section 07 and [SGL] "DSpark：sequential head 加验证预算": the confidence head
    is trained on one minus the total-variation distance between the drafter's and the
    target's distributions at that position.
    """
    return 1.0 - 0.5 * float(np.sum(np.abs(np.asarray(p_d) - np.asarray(p_t))))


def accept_request_capped(target_rows, draft_rows, tokens, u_accept, u_resample, cap):
    """Cap-accept verify mode for one request.

    [SGL] "Confidence scheduler 与 verify 模式" and [CSDN] section 5: the whole drafted block
    is verified (as in static mode) but only positions inside the scheduler's window may be
    committed, so the commit is the one compact mode makes for that window, while the
    acceptance the whole block would have reached -- the ceiling the trimming gave up -- is
    recorded as well.

    ``target_rows`` [w, V] are the target logits of the whole verified block (w rows,
    anchor included), ``draft_rows`` [w-1, V]; ``cap`` in [1, w] is the window.

    * n_full: accepted drafts over the whole block (first rejection among drafts 1..w-1);
    * committed drafts n = min(n_full, cap - 1);
    * y: when the block rejects inside the window (n_full < cap - 1) the residual draw of
      that rejection, otherwise the bonus draw from p_t of row cap - 1 -- compact mode's
      draw for the window cap;
    * labels, p_t(x), p_d(x) for every draft of the block.
    Returns the ``accept_request`` fields plus ``n_full``.
    """
    w = len(target_rows)
    cap = int(cap)
    assert 1 <= cap <= w
    p_t = [softmax64(r) for r in target_rows]
    p_d = [softmax64(r) for r in draft_rows]
    pt_at = [float(p_t[k - 1][int(tokens[k - 1])]) for k in range(1, w)]
    pd_at = [float(p_d[k - 1][int(tokens[k - 1])]) for k in range(1, w)]
    labels = [tv_label(p_d[k - 1], p_t[k - 1]) for k in range(1, w)]
    margins = []
    n_full = w - 1
    for k in range(1, w):  # the whole block, as the full verify sees it
        pt, pd = pt_at[k - 1], pd_at[k - 1]
        r = np.inf if pd == 0.0 else pt / pd
        u = float(np.float32(u_accept[k - 1]))
        margins.append(abs(u - r))
        if not u < min(1.0, r):
            n_full = k - 1
            break
    n = min(n_full, cap - 1)
    if n_full < cap - 1:  # rejected inside the window: residual of that pair
        dist = np.maximum(0.0, p_t[n] - p_d[n])
        if not np.sum(dist) > 0.0:
            dist = p_t[n]
    else:  # the window's drafts all survive: bonus from the window's last target row
        dist = p_t[cap - 1]
    y, draw_margin = inverse_cdf(dist, float(np.float32(u_resample)))
    committed = [int(tokens[i]) for i in range(n)] + [y]
    return {"n": n, "n_full": n_full, "committed": committed, "margins": margins,
            "draw_margin": draw_margin, "labels": labels, "pt_at": pt_at, "pd_at": pd_at}


def accept_and_commit(target_logits, draft_logits, draft_tokens, u_accept, u_resample,
                      windows, cu_seqlens, context_lens):
    """Batch driver: one ``accept_request`` per request, then the commit bookkeeping.

    target_logits [R, V] packed rows; draft_logits [B, gamma-1, V]; draft_tokens,
    u_accept [B, gamma-1]; u_resample [B]; windows [B]; cu_seqlens [B+1];
    context_lens [B].

    Commit ([NOTES] sections 02 and 09): the anchor and the n accepted drafts now have
    valid KV, and the drawn token y becomes the next anchor, so
    ``context_lens[b] += n + 1``; rejected positions are dropped simply by not advancing
    past them.  ``committed[b, :n+1]`` holds ``x_1 .. x_n, y``; the rest is -1.
    Labels and the per-draft probabilities are reported for every verified draft
    (k < w); entries outside the window are NaN.
    """
    draft_tokens = np.asarray(draft_tokens)
    B, G = draft_tokens.shape
    gamma = G + 1
    accept_len = np.zeros(B, dtype=np.int32)
    committed = np.full((B, gamma), -1, dtype=np.int32)
    new_ctx = np.asarray(context_lens, dtype=np.int64).copy()
    labels = np.full((B, G), np.nan, dtype=np.float64)
    pt_at = np.full((B, G), np.nan, dtype=np.float64)
    pd_at = np.full((B, G), np.nan, dtype=np.float64)
    margins = []
    draw_margins = np.zeros(B, dtype=np.float64)
    for b in range(B):
        w = int(windows[b])
        r0 = int(cu_seqlens[b])
        res = accept_request(target_logits[r0:r0 + w], draft_logits[b, : w - 1],
                             draft_tokens[b, : w - 1], u_accept[b, : w - 1], u_resample[b])
        accept_len[b] = res["n"]
        committed[b, : res["n"] + 1] = res["committed"]
        new_ctx[b] += res["n"] + 1
        labels[b, : w - 1] = res["labels"]
        pt_at[b, : w - 1] = res["pt_at"]
        pd_at[b, : w - 1] = res["pd_at"]
        margins.append(res["margins"])
        draw_margins[b] = res["draw_margin"]
    return {"accept_len": accept_len, "committed": committed,
            "context_lens": new_ctx.astype(np.int32), "labels": labels, "pt_at": pt_at,
            "pd_at": pd_at, "margins": margins, "draw_margins": draw_margins}


def confidence_labels(target_logits, draft_logits, windows, cu_seqlens):
    """Stage 5 on its own: ``labels[b, k-1] = c*`` for draft k < w_b, NaN elsewhere."""
    B = len(windows)
    G = np.asarray(draft_logits).shape[1]
    labels = np.full((B, G), np.nan, dtype=np.float64)
    for b in range(B):
        w = int(windows[b])
        r0 = int(cu_seqlens[b])
        for k in range(1, w):
            labels[b, k - 1] = tv_label(softmax64(draft_logits[b, k - 1]),
                                        softmax64(target_logits[r0 + k - 1]))
    return labels
