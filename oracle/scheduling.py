"""Oracle for stage 1: confidence head, prefix survival and the window scheduler.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product path.

Window convention used throughout the path: a block holds ``gamma`` positions.  Position 0
is the anchor (the last committed token, whose target row verifies the first draft); the
other ``gamma - 1`` positions are drafts and carry a confidence each.  A request's window
``w`` counts packed verify rows, anchor included, so ``w`` is in ``[1, gamma]`` and the
request verifies ``w - 1`` drafts.  This is the reading under which the tier example of
[SGL] "Ragged verify under full CUDA graphs" (windows 5/3/2 give 10 rows, tier 12), the
cost model of [CSDN] section 4 (M = bs + K with K the extra verify tokens) and the
five-row survival table of [NOTES] section 07 (block length 6) agree.
"""

from __future__ import annotations

import numpy as np


def confidence_from_head(hidden, head_w, head_b, sts_T=None):
    """Confidence head + Sequential Temperature Scaling.

    [SGL] "DSpark：sequential head 加验证预算" and [NOTES] section 07: the confidence head
    is one linear layer followed by a sigmoid on the drafter hidden state, one score per
    draft position.  [NOTES] section 07 ("为什么还要做 Sequential Temperature Scaling")
    calibrates the scores per position with a temperature.  Reading: the temperature
    divides the head's logit before the sigmoid, ``c_k = sigmoid(z_k / T_k)``; ``T_k = 1``
    (or ``sts_T is None``) is the identity.

    hidden: [B, gamma-1, H] (bf16 or fp32 values, any float dtype); head_w: [H];
    head_b: scalar (treated as float32); sts_T: [gamma-1] or None.
    Math in float64, result rounded once to float32.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(head_w, dtype=np.float32).astype(np.float64)
    b0 = float(np.float32(head_b))
    B, G, H = h.shape
    z = np.empty((B, G), dtype=np.float64)
    for b in range(B):
        for k in range(G):
            z[b, k] = float(np.dot(h[b, k], w)) + b0
    if sts_T is not None:
        T = np.asarray(sts_T, dtype=np.float32).astype(np.float64)
        z = z / T[None, :]
    c = 1.0 / (1.0 + np.exp(-z))
    return c.astype(np.float32)


def survival(c):
    """Prefix survival ``a_j = prod_{i<=j} c_i`` per request.

    [NOTES] section 07 ("从单点置信度到前缀存活概率"): acceptance keeps a contiguous
    prefix, so the probability that draft j is still alive is the product of the
    conditional scores up to j.  The product is formed left to right in float32, one
    IEEE multiply per step (no fused operations), so that a GPU doing the same sequence of
    float32 multiplies agrees bit for bit.
    """
    c = np.asarray(c, dtype=np.float32)
    a = np.empty_like(c)
    B, G = c.shape
    for b in range(B):
        a[b, 0] = c[b, 0]
        for j in range(1, G):
            a[b, j] = np.float32(a[b, j - 1] * c[b, j])
    return a


def step_cost(bias, alpha, theta, bs, K):
    """Additive step-cost model ``T(bs, K) = bias + alpha(bs) + theta(bs + K)``.

    [CSDN] section 4: alpha(bs) is the per-request floor that trimming cannot recover;
    theta(M) with M = bs + K is the verify-token cost.  Tables hold float32 milliseconds;
    the sum is formed in float64 left to right.
    """
    return (float(np.float32(bias)) + float(np.float32(alpha[bs]))) + float(np.float32(theta[bs + K]))


def schedule_windows(a, gamma, bias, alpha, theta, static=False, tie_rtol=1e-9):
    """Hardware-aware prefix scheduler: one verify window per request.

    [NOTES] section 08 ("8.3 调度器在优化什么？"): candidates (request, position) are
    ranked by prefix survival and added while expected throughput
    (expected accepted tokens x steps per second) keeps rising; [CSDN] section 4 states
    the same choice as an argmax against the measured cost T(bs, K).  Reading used here:

    * expected tokens after adding the K best candidates: ``E_K = B + S_K`` (every request
      also gets its bonus/correction token), ``S_K`` the float64 sum of the K largest
      survivals taken in rank order;
    * rank order: survival descending, then request ascending, then position ascending;
    * ``K* = argmax_K E_K / T(B, K)`` over ``K = 0 .. B(gamma-1)``, smallest K on a tie;
    * window ``w_b = 1 + (number of request b's candidates among the first K*)``.

    ``static=True`` is the full-block comparison arm: every window is ``gamma``.

    Returns dict(windows [B] int32, K, ratio, ratios [N+1] float64, near_tie bool).
    ``near_tie`` flags another K whose ratio is within ``tie_rtol`` (relative) of the best.
    """
    a = np.asarray(a, dtype=np.float32)
    B, G = a.shape
    assert G == gamma - 1
    N = B * G
    cands = []
    for b in range(B):
        for j in range(G):
            cands.append((-float(a[b, j]), b, j))
    cands.sort()
    E = float(B)
    ratios = np.empty(N + 1, dtype=np.float64)
    for K in range(N + 1):
        if K > 0:
            E = E + (-cands[K - 1][0])
        T = step_cost(bias, alpha, theta, B, K)
        if not T > 0.0:
            raise ValueError("step cost must be positive")
        ratios[K] = E / T
    if static:
        Kstar = N
    else:
        Kstar = 0
        for K in range(1, N + 1):
            if ratios[K] > ratios[Kstar]:
                Kstar = K
    windows = np.ones(B, dtype=np.int32)
    for i in range(Kstar):
        windows[cands[i][1]] += 1
    best = ratios[Kstar]
    near_tie = False
    if not static:
        for K in range(N + 1):
            if K != Kstar and abs(ratios[K] - best) <= tie_rtol * abs(best):
                near_tie = True
    return {"windows": windows, "K": int(Kstar), "ratio": float(best), "ratios": ratios,
            "near_tie": near_tie}

