"""Host logic of the measured step-cost tables (CPU only).

The additive model T(bs, K) = bias + alpha(bs) + theta(bs + K) of the devpress.csdn.net
article on DSpark in SGLang (section "4. 零开销调度如何隐藏计算成本") is fitted from
measured step times; these tests pin the fit on synthetic times with known parameters, and
pin what a tier-step theta does to the scheduler's choice (the oracle's argmax).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from ragged_verify_acceptance_amd.costmodel import (even_windows, fit_additive, fit_linear,
                                                    scheduler_tables, tier_of)
from workloads.costgrid import grid_points

TIERS = tuple(range(8, 513, 8))


def _synthetic(bs_list, gamma, alpha_fn, theta_tier, noise=0.0, seed=0):
    rng = np.random.default_rng(seed)
    out = []
    for bs in bs_list:
        for M in grid_points(bs, gamma, TIERS):
            t = alpha_fn(bs) + theta_tier[tier_of(M, TIERS)] + noise * rng.standard_normal()
            out.append((bs, M, t))
    return out


def test_tier_of_and_windows():
    assert tier_of(1, TIERS) == 8 and tier_of(8, TIERS) == 8 and tier_of(9, TIERS) == 16
    with pytest.raises(ValueError):
        tier_of(513, TIERS)
    for bs, M in [(1, 1), (1, 8), (5, 17), (64, 308), (64, 512)]:
        w = even_windows(bs, M, 8)
        assert w.sum() == M and w.min() >= 1 and w.max() <= 8 and w.max() - w.min() <= 1
    with pytest.raises(ValueError):
        even_windows(4, 3, 8)
    assert grid_points(4, 8, TIERS) == [4, 8, 16, 24, 32]
    assert grid_points(64, 8, TIERS)[:3] == [64, 72, 80] and grid_points(64, 8, TIERS)[-1] == 512


def test_fit_recovers_known_tables():
    rng = np.random.default_rng(3)
    theta = {t: 0.0 for t in TIERS}
    acc = 0.0
    for t in TIERS:
        theta[t] = acc
        acc += float(rng.uniform(0.1, 2.0))   # non-decreasing step cost
    bs_list = [1, 2, 4, 8, 16, 32, 48, 64]
    alpha = {bs: 5.0 + 3.1 * bs + float(rng.uniform(0, 1)) for bs in bs_list}
    s = _synthetic(bs_list, 8, lambda b: alpha[b], theta)
    f = fit_additive(s, TIERS)
    assert f.rms < 1e-9 and f.max_abs < 1e-9
    t0 = f.tiers[0]
    for i, t in enumerate(f.tiers):
        assert abs(f.theta[i] - (theta[t] - theta[t0])) < 1e-9
    for i, b in enumerate(f.bs):
        assert abs(f.alpha[i] - (alpha[b] + theta[t0])) < 1e-9
    # with noise the fit stays close and reports a residual of the noise's size
    fn = fit_additive(_synthetic(bs_list, 8, lambda b: alpha[b], theta, noise=0.05), TIERS)
    assert 0.02 < fn.rms < 0.08
    assert np.max(np.abs(fn.theta - f.theta)) < 0.2


def test_fit_linear_recovers_slope():
    s = [(bs, M, 7.0 + 2.0 * bs + 0.25 * M) for bs in (1, 4, 16) for M in range(bs, 8 * bs + 1)]
    bs, alpha, th1, rms = fit_linear(s)
    assert abs(th1 - 0.25) < 1e-12 and rms < 1e-9
    assert np.allclose(alpha, [9.0, 15.0, 39.0])


def test_fit_rejects_unlinked_batch_sizes():
    # bs = 1 only reaches tier 8, bs = 64 only tiers >= 64: alpha(64) and theta(tiers >= 64)
    # trade off freely, so the split is undetermined
    s = [(1, M, 1.0) for M in range(1, 9)] + [(64, M, 2.0 + M) for M in range(64, 513, 8)]
    with pytest.raises(ValueError):
        fit_additive(s, TIERS)


def test_scheduler_tables_shape():
    theta = {t: 0.01 * t for t in TIERS}
    f = fit_additive(_synthetic([1, 2, 4, 8, 16], 8, lambda b: 10 + b, theta), TIERS)
    bias, alpha, th = scheduler_tables(f, 16, 8, TIERS)
    assert bias == 0.0 and alpha.shape == (17,) and th.shape == (129,)
    assert alpha.dtype == np.float32 and th.dtype == np.float32
    for t_lo, t_hi in zip((0,) + TIERS, TIERS):
        if t_hi > 128:
            break
        seg = th[t_lo + 1: t_hi + 1]
        assert np.all(seg == seg[0])            # constant inside a tier
    assert abs(alpha[3] - 0.5 * (alpha[2] + alpha[4])) < 1e-5  # interpolated between measured bs


@pytest.mark.parametrize("seed", range(40))
def test_tier_step_cost_stops_at_tier_end(seed):
    """With theta constant inside each tier, expected tokens rise with every added candidate
    while the cost stays flat, so the argmax never stops inside a tier: the chosen row count
    is a tier value or the whole batch."""
    rng = np.random.default_rng(seed)
    B, gamma = int(rng.integers(2, 17)), int(rng.integers(3, 9))
    tiers = tuple(range(4, B * gamma + 4, 4))
    c = rng.beta(4, 1, size=(B, gamma - 1)).astype(np.float32)
    a = oracle.survival(c)
    step = rng.uniform(0.05, 3.0)
    theta = np.array([0.0] + [step * tier_of(M, tiers) for M in range(1, B * gamma + 1)], np.float32)
    alpha = np.zeros(B + 1, np.float32)
    r = oracle.schedule_windows(a, gamma, np.float32(rng.uniform(1, 30)), alpha, theta)
    M = int(np.sum(r["windows"]))
    assert M == B * gamma or M == tier_of(M, tiers) or r["near_tie"]
