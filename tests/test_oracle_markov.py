"""Pins for the oracle's Markov sequential head (CPU only).  Each test names the mistake it
would catch."""

import numpy as np
import pytest
import torch

import oracle
from oracle.markov import markov_bias
from workloads.generate import markov_inputs


def _softmax_np(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def test_bias_is_the_exact_integer_product():
    """Brute force with Python integers and exact rationals on a tiny vocabulary: the bias is
    (s1[x] s2[v]) * sum_j q1[x,j] q2[v,j].  Catches a transposed factor (q2[:, v]), a
    missing scale, or the scale of v used for x."""
    from fractions import Fraction

    inp = markov_inputs(1, 1, 1, 24, r=16)
    q1, q2, s1, s2 = inp["q1"], inp["q2"], inp["s1"], inp["s2"]
    x = 5
    b = markov_bias(q1[x], s1[x], q2.astype(np.float64), s2)
    for v in range(24):
        dot = sum(int(q1[x, j]) * int(q2[v, j]) for j in range(16))
        exact = Fraction(float(s1[x])) * Fraction(float(s2[v])) * dot
        assert abs(Fraction(float(b[v])) - exact) <= abs(exact) * Fraction(1, 2 ** 52)


def test_zero_bias_is_independent_sampling():
    """With zero weights every position is an independent inverse-CDF draw from softmax(U_k)
    (numpy's searchsorted on the cumulative sum), whatever the anchor.  Catches a draw from
    the wrong row, a descending-order CDF, or a strict/loose inequality swap."""
    inp = markov_inputs(2, 3, 4, 50, r=8, dtype="f32")
    z = np.zeros_like(inp["q1"])
    r = oracle.markov_sample(inp["U"], inp["anchor"], inp["u"], z, inp["s1"], z, inp["s2"])
    for b in range(3):
        for k in range(4):
            p = _softmax_np(inp["U"][b, k].double().numpy())
            y = int(np.searchsorted(np.cumsum(p), float(inp["u"][b, k]) * np.sum(p), side="right"))
            assert r["tokens"][b, k] == y
            assert abs(r["p_at"][b, k] - p[y]) < 1e-12
    assert torch.equal(r["logits"], inp["U"])


def test_transition_chain_follows_previous_token():
    """A bias that makes token (x+1) mod V overwhelmingly likely after x: the block is the
    chain anchor+1, anchor+2, ...  Catches conditioning on the wrong position (x_k instead
    of x_{k-1}, or the anchor ignored)."""
    V, r, G1 = 16, 16, 6
    q1 = np.zeros((V, r), np.int8)
    q2 = np.zeros((V, r), np.int8)
    for x in range(V):
        q1[x, x] = 100                 # one-hot embedding of x
        q2[(x + 1) % V, x] = 100       # projection onto the successor
    s = np.full(V, 0.01, np.float32)   # bias = 0.01 * 0.01 * 10000 = 1 ... scaled below
    s2 = np.full(V, 0.5, np.float32)   # bias(x, x+1) = 0.01 * 0.5 * 10000 = 50
    U = torch.zeros((2, G1, V), dtype=torch.float32)
    anchor = np.array([3, 15], np.int32)
    u = np.full((2, G1), 0.5, np.float32)
    out = oracle.markov_sample(U, anchor, u, q1, s, q2, s2)
    assert out["tokens"][0].tolist() == [(3 + k) % V for k in range(1, G1 + 1)]
    assert out["tokens"][1].tolist() == [(15 + k) % V for k in range(1, G1 + 1)]


def test_empirical_distribution_matches_softmax():
    """Over many uniforms the tokens drawn at position 1 follow softmax(U_1 + B(anchor, .))
    (chi-square, V = 8).  Catches a bias of the wrong sign or a sampling rule that is not
    the distribution."""
    from scipy.stats import chisquare

    inp = markov_inputs(3, 1, 1, 8, r=8, dtype="f32")
    n = 20000
    rng = np.random.default_rng(0)
    U = inp["U"].expand(n, 1, 8).contiguous()
    anchor = np.full(n, int(inp["anchor"][0]), np.int32)
    u = rng.random((n, 1), dtype=np.float32)
    out = oracle.markov_sample(U, anchor, u, inp["q1"], inp["s1"], inp["q2"], inp["s2"])
    x = int(inp["anchor"][0])
    p = _softmax_np(inp["U"][0, 0].double().numpy()
                    + (float(inp["s1"][x]) * inp["s2"].astype(np.float64))
                    * (inp["q2"].astype(np.int64) @ inp["q1"][x].astype(np.int64)))
    counts = np.bincount(out["tokens"][:, 0], minlength=8)
    keep = p * n > 5
    assert chisquare(counts[keep], p[keep] / p[keep].sum() * counts[keep].sum()).pvalue > 1e-3


def test_stored_logits_are_bf16_of_the_float64_sum():
    """bfloat16 storage: the stored logit is the float64 value rounded (to float32, then to
    bfloat16); values that bfloat16 holds exactly are stored exactly."""
    V, r = 8, 4
    q1 = np.zeros((V, r), np.int8)
    q2 = np.zeros((V, r), np.int8)
    q1[0, 0] = 2
    q2[:, 0] = np.arange(V)
    s1 = np.full(V, 0.5, np.float32)
    s2 = np.full(V, 0.25, np.float32)     # bias(0, v) = 0.5 * 0.25 * 2 v = v / 4
    U = torch.full((1, 1, V), 1.0, dtype=torch.bfloat16)
    out = oracle.markov_sample(U, np.array([0]), np.array([[0.3]], np.float32), q1, s1, q2, s2)
    assert out["logits"][0, 0].float().tolist() == [1.0 + v / 4 for v in range(V)]
