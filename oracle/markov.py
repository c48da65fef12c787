"""Markov sequential head: per-position logits with a first-order transition bias, sampled
in sequence.

TEST INFRASTRUCTURE (part of the CPU oracle package; see ``oracle/__init__.py``).

Sources:

* [NOTES] section "05 · Core Innovation A" (semi-autoregressive generation), 5.1-5.3: the parallel
  backbone gives base logits U_1 .. U_gamma for the whole block in one pass; the
  sequential head adds a prefix-dependent bias, p_k(v | x_<k) proportional to
  exp(U_k(v) + B_k(prefix, v)); the Markov head's bias depends on the previous token only,
  B(x_{k-1}, v), stored as a rank-r product W1 W2 (r = 256 by default), so a step is an
  embedding lookup and a projection.  Section 09: the light sequential module samples the
  positions in order.
* [SGL] "DSpark：sequential head 加验证预算": each position is conditioned on the one
  before it ("semi-autoregressive").

Readings (the pages fix neither precision nor sampling details):

* Position k = 1 .. gamma-1 of request b is conditioned on x_{k-1}, with x_0 the anchor
  (the last committed token).
* Weights are stored as int8 with float32 scales: W1 rows ``q1[x, :]`` with scale
  ``s1[x]`` (the embedding of the previous token) and W2 as vocabulary rows ``q2[v, :]``
  with scale ``s2[v]``, so the bias is
  ``B(x, v) = (s1[x] * s2[v]) * sum_j q1[x, j] q2[v, j]``, the integer dot product exact.
  The logit is formed in float64 as ``U_k(v) + ((s1[x] * s2[v]) * dot)`` (the scale
  product exact, then one rounded multiply and one rounded add, no fused operation) and
  stored in the dtype of U (bfloat16: rounded to float32, then to bfloat16, both to
  nearest even).
* The token is drawn from the STORED logits (these are the draft distribution the
  acceptance step compares against), at temperature 1, by the inverse CDF in ascending
  token order with the position's uniform (as ``inverse_cdf``).
"""

from __future__ import annotations

import numpy as np
import torch

from .acceptance import inverse_cdf


def markov_bias(q1_row, s1_x, q2f, s2):
    """float64 [V]: (s1[x] * s2[v]) * (q1[x] . q2[v]) for every v.  ``q2f`` is q2 as
    float64: every partial sum of int8 x int8 products over r <= 2^16 terms is an integer
    below 2^53, so the float64 matrix-vector product is the exact integer dot product in
    any summation order."""
    dot = q2f @ q1_row.astype(np.float64)
    t = np.float64(np.float32(s1_x)) * s2.astype(np.float32).astype(np.float64)  # exact
    return t * dot


def store_logits(l64, dtype):
    """Round float64 logits to the storage dtype ("bf16": via float32, both RNE)."""
    f32 = torch.from_numpy(np.asarray(l64, np.float64)).to(torch.float32)
    return f32.to(torch.bfloat16) if dtype == "bf16" else f32


def markov_sample(U, anchor, u, q1, s1, q2, s2):
    """Sequential sampling of one block per request.

    U: [B, G1, V] torch tensor (bfloat16 or float32) of base logits for positions 1..G1;
    anchor [B] int; u [B, G1] float32; q1, q2 [V, r] int8; s1, s2 [V] float32.
    Returns dict(tokens int32 [B, G1], logits torch [B, G1, V] (U's dtype),
    p_at float64 [B, G1] (probability of the drawn token), margins float64 [B, G1]
    (distance of the draw to its bin edges relative to the total mass)."""
    dtype = "bf16" if U.dtype == torch.bfloat16 else "f32"
    B, G1, V = U.shape
    q1 = np.asarray(q1, np.int8)
    q2f = np.asarray(q2, np.int8).astype(np.float64)
    s1 = np.asarray(s1, np.float32)
    s2 = np.asarray(s2, np.float32)
    tokens = np.zeros((B, G1), np.int32)
    p_at = np.zeros((B, G1))
    margins = np.zeros((B, G1))
    logits = torch.empty((B, G1, V), dtype=U.dtype)
    for b in range(B):
        x = int(anchor[b])
        for k in range(G1):
            l64 = U[b, k].double().numpy() + markov_bias(q1[x], s1[x], q2f, s2)
            stored = store_logits(l64, dtype)
            logits[b, k] = stored
            ls = stored.double().numpy()
            e = np.exp(ls - np.max(ls))
            y, m = inverse_cdf(e, float(np.float32(u[b, k])))
            tokens[b, k] = y
            p_at[b, k] = e[y] / np.sum(e)
            margins[b, k] = m
            x = y
    return {"tokens": tokens, "logits": logits, "p_at": p_at, "margins": margins}
