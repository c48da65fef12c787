"""Step-cost tables for the window scheduler, fitted from measured step times.

The scheduler's cost model is additive (the devpress.csdn.net article on DSpark in SGLang,
section "4. 零开销调度如何隐藏计算成本"): T(bs, K) = bias + alpha(bs) + theta(M) with M = bs + K, where
alpha is the per-request floor that pruning does not touch and theta the cost of the verify
tokens.  Given step times measured at a grid of (bs, M), ``fit_additive`` finds alpha per
measured bs and theta per padded tier (the graph that runs M rows pads them to tier(M), so
the cost the scheduler should see is a step function of M); ``fit_linear`` gives the plain
per-token slope for comparison.  ``scheduler_tables`` expands a fit into the arrays the
scheduling call takes (alpha indexed by bs, theta indexed by M).

Host-side least squares on a few hundred numbers; nothing here runs on the path.
"""

from __future__ import annotations

from bisect import bisect_left
from dataclasses import dataclass

import numpy as np


def tier_of(M: int, tiers) -> int:
    """Smallest tier >= M (the padded row count the step runs)."""
    i = bisect_left(list(tiers), M)
    if i == len(tiers):
        raise ValueError(f"M={M} exceeds the largest tier {tiers[-1]}")
    return int(tiers[i])


@dataclass
class AdditiveFit:
    bs: np.ndarray          # measured batch sizes, ascending
    alpha: np.ndarray       # alpha(bs) for those, same units as the measurements
    tiers: np.ndarray       # tiers with a theta (every tier some measurement fell in)
    theta: np.ndarray       # theta(tier), theta of the smallest tier = 0
    rms: float              # root-mean-square residual of the fit
    max_abs: float          # largest absolute residual


def fit_additive(samples, tiers) -> AdditiveFit:
    """Least-squares fit of T(bs, M) = alpha(bs) + theta(tier(M)).

    ``samples``: iterable of (bs, M, T).  The bias is folded into alpha (only the sum
    enters the scheduler) and theta is anchored at 0 on the smallest observed tier.  Every
    measured bs must share a tier with another one through a chain of overlapping M ranges,
    or the split between alpha and theta is not determined (then ValueError)."""
    s = [(int(b), int(m), float(t)) for b, m, t in samples]
    if not s:
        raise ValueError("no samples")
    bs = np.array(sorted({b for b, _, _ in s}))
    ts = np.array(sorted({tier_of(m, tiers) for _, m, _ in s}))
    nb, nt = len(bs), len(ts)
    A = np.zeros((len(s), nb + nt - 1))
    y = np.zeros(len(s))
    for i, (b, m, t) in enumerate(s):
        A[i, int(np.searchsorted(bs, b))] = 1.0
        k = int(np.searchsorted(ts, tier_of(m, tiers)))
        if k > 0:
            A[i, nb + k - 1] = 1.0
        y[i] = t
    if np.linalg.matrix_rank(A) < A.shape[1]:
        raise ValueError("alpha(bs) and theta(tier) are not separable on these samples")
    x, *_ = np.linalg.lstsq(A, y, rcond=None)
    r = y - A @ x
    return AdditiveFit(bs=bs, alpha=x[:nb], tiers=ts, theta=np.concatenate([[0.0], x[nb:]]),
                       rms=float(np.sqrt(np.mean(r * r))), max_abs=float(np.max(np.abs(r))))


def fit_linear(samples):
    """Least-squares fit of T(bs, M) = alpha(bs) + theta1 * M; returns (bs, alpha, theta1, rms)."""
    s = [(int(b), int(m), float(t)) for b, m, t in samples]
    bs = np.array(sorted({b for b, _, _ in s}))
    A = np.zeros((len(s), len(bs) + 1))
    y = np.zeros(len(s))
    for i, (b, m, t) in enumerate(s):
        A[i, int(np.searchsorted(bs, b))] = 1.0
        A[i, -1] = m
        y[i] = t
    x, *_ = np.linalg.lstsq(A, y, rcond=None)
    r = y - A @ x
    return bs, x[:-1], float(x[-1]), float(np.sqrt(np.mean(r * r)))


def scheduler_tables(fit: AdditiveFit, B: int, gamma: int, tiers):
    """(bias, alpha [B+1], theta [B*gamma+1]) float32 for the scheduling call.

    alpha at an unmeasured bs is interpolated linearly in bs (held flat outside the measured
    range); theta[M] = theta(tier(M)), held at the nearest fitted tier for tiers the
    measurements did not reach.  bias = 0 (it is folded into alpha)."""
    alpha = np.interp(np.arange(B + 1), fit.bs, fit.alpha).astype(np.float32)
    theta = np.zeros(B * gamma + 1, np.float32)
    for M in range(1, B * gamma + 1):
        t = tier_of(M, tiers)
        k = min(int(np.searchsorted(fit.tiers, t)), len(fit.tiers) - 1)
        theta[M] = fit.theta[k]
    return np.float32(0.0), alpha, theta


def even_windows(bs: int, M: int, gamma: int) -> np.ndarray:
    """Windows (anchor included, each in [1, gamma]) of bs requests that sum to M, as even as
    possible (the first M mod bs requests get one more)."""
    if not bs <= M <= bs * gamma:
        raise ValueError(f"M={M} outside [{bs}, {bs * gamma}]")
    w = np.full(bs, M // bs, np.int32)
    w[: M % bs] += 1
    return w
