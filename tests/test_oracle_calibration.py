"""Pins for the oracle's Sequential Temperature Scaling fit and ECE (CPU only).

Each test names the mistake it would catch.
"""

import numpy as np
import pytest

import oracle
from oracle.calibration import position_nll
from workloads.generate import calibration_trace


def _z_of(p):
    p = np.asarray(p, dtype=np.float64)
    return np.log(p / (1 - p)).astype(np.float32)


# ---------------------------------------------------------------- ECE


def test_ece_hand_example():
    """Two bins: {0.2, 0.3} with outcomes {0, 1}, {0.8, 0.9} with {1, 1}:
    0.5 * |0.25 - 0.5| + 0.5 * |0.85 - 1| = 0.2.  Catches unweighted bin averages,
    squared gaps, or bins of the outcome instead of the prediction."""
    z = _z_of([0.2, 0.3, 0.8, 0.9])[:, None]
    n = np.array([0, 1, 1, 1])
    r = oracle.ece(z, n, n_bins=2)
    assert abs(r["pooled"] - 0.2) < 1e-6
    assert r["counts"].tolist() == [[2, 2]] and r["sum_e"].tolist() == [[1, 2]]


def test_ece_calibrated_and_constant():
    """A constant prediction p against outcome frequency f gives |p - f|; p = f gives 0."""
    z = np.full((8, 1), _z_of([0.75])[0])
    assert oracle.ece(z, np.array([1, 1, 1, 0] * 2), n_bins=10)["pooled"] < 1e-6
    r = oracle.ece(z, np.array([1, 0, 0, 0] * 2), n_bins=10)
    assert abs(r["pooled"] - 0.5) < 1e-6


def test_ece_uses_prefix_survival_and_positions():
    """Position 2's prediction is sigmoid(z1) * sigmoid(z2), its outcome [n >= 2]; the pooled
    value weights the positions by their counts.  Catches per-position scores used
    unmultiplied, or the outcome of position k taken as [n == k]."""
    z = np.tile(_z_of([0.9, 0.5]), (4, 1))       # a = 0.9, 0.45
    n = np.array([2, 1, 0, 2])                   # E1 = 1,1,0,1; E2 = 1,0,0,1
    r = oracle.ece(z, n, n_bins=10)
    assert abs(r["per_position"][0] - abs(0.9 - 0.75)) < 1e-6
    assert abs(r["per_position"][1] - abs(0.45 - 0.5)) < 1e-6
    assert abs(r["pooled"] - 0.5 * (0.15 + 0.05)) < 1e-6


def test_ece_ignores_unobserved_positions():
    """Samples whose positions were never verified (compact windows) change nothing."""
    z, n, _ = calibration_trace(5, 300, 4, 1.5)
    base = oracle.ece(z, n)
    z2 = np.concatenate([z, z[:50] * 3.0])
    n2 = np.concatenate([n, np.zeros(50, np.int32)])
    o2 = np.concatenate([np.full(300, 4, np.int32), np.zeros(50, np.int32)])
    r = oracle.ece(z2, n2, observed_len=o2)
    assert r["pooled"] == base["pooled"]
    assert np.array_equal(r["per_position"], base["per_position"])


# ---------------------------------------------------------------- STS fit


def test_single_position_is_temperature_scaling():
    """With one draft position the fit is logistic regression on z without an intercept:
    1/T equals scikit-learn's unpenalised coefficient.  Catches z * T instead of z / T,
    a sign error, or a wrong likelihood."""
    from sklearn.linear_model import LogisticRegression

    z, n, _ = calibration_trace(11, 4000, 1, 1.7, noise=0.3)
    r = oracle.sts_fit(z, n, grid=257)
    lr = LogisticRegression(fit_intercept=False, penalty=None, tol=1e-12, max_iter=10000)
    lr.fit(z.astype(np.float64), n >= 1)
    assert abs(1.0 / r["T64"][0] - lr.coef_[0, 0]) < 1e-5 * abs(lr.coef_[0, 0])


@pytest.mark.parametrize("T_true", [[1.0, 1.0, 1.0, 1.0], [1.5, 2.0, 0.7, 1.2]])
def test_recovers_known_temperatures(T_true):
    """Traces drawn with a known over/under-confidence: the fit recovers it.  Catches a fit
    that ignores the earlier positions' survival (it would bias the later temperatures)."""
    z, n, _ = calibration_trace(21, 20000, 4, T_true, beta=(5.0, 1.5))
    r = oracle.sts_fit(z, n, grid=257)
    assert np.all(np.abs(r["T64"] / np.array(T_true) - 1) < 0.08), r["T64"]
    # a fit that drops the prefix (each position alone against [n >= k]) misses
    obs, E = oracle.calibration.observed_outcomes(n, None, 4)
    zero = np.zeros(len(n))
    u = np.linspace(np.log(0.05), np.log(20), 801)
    f = [position_nll(z[:, 3].astype(np.float64), zero, E[:, 3], obs[:, 3], np.exp(x)) for x in u]
    T_alone = np.exp(u[int(np.argmin(f))])
    assert abs(T_alone / T_true[3] - 1) > 0.2


def test_censored_trace_still_recovers():
    """Compact-mode traces observe only the window's positions; the fit uses what was
    observed and still recovers the temperatures."""
    T_true = [1.4, 1.8, 2.2]
    z, n, o = calibration_trace(31, 30000, 3, T_true, beta=(5.0, 1.5), censor=True)
    n = np.minimum(n, o)   # a censored run cannot report acceptance past its window
    r = oracle.sts_fit(z, n, observed_len=o, grid=257)
    assert np.all(np.abs(r["T64"] / np.array(T_true) - 1) < 0.1), r["T64"]
    assert np.all(r["n_obs"] < 30000)


def test_fit_is_a_minimum_and_sequential():
    """The fitted temperature is a local minimum of its position's likelihood, and adding a
    later position leaves the earlier temperatures unchanged."""
    z, n, _ = calibration_trace(41, 3000, 3, [1.3, 1.6, 1.9], noise=0.5)
    r = oracle.sts_fit(z, n, grid=257)
    obs, E = oracle.calibration.observed_outcomes(n, None, 3)
    L = np.zeros(len(n))
    for k in range(3):
        f0 = position_nll(z[:, k].astype(np.float64), L, E[:, k], obs[:, k], r["T64"][k])
        for eps in (1e-4, -1e-4):
            assert position_nll(z[:, k].astype(np.float64), L, E[:, k], obs[:, k],
                                r["T64"][k] * (1 + eps)) >= f0
        assert abs(f0 - r["nll"][k]) < 1e-9 * f0
        L = L + oracle.log_prefix_survival(z[:, k:k + 1], r["T"][k:k + 1])[:, 0]
    r2 = oracle.sts_fit(z[:, :2], np.minimum(n, 2), grid=257)
    assert np.allclose(r2["T64"], r["T64"][:2], rtol=1e-9)


def test_calibration_lowers_ece():
    """An over-confident head (T = 2) is miscalibrated; after the fit its ECE drops."""
    z, n, _ = calibration_trace(51, 8000, 5, 2.0, noise=0.2)
    before = oracle.ece(z, n)["pooled"]
    r = oracle.sts_fit(z, n, grid=257)
    after = oracle.ece(z, n, T=r["T"])["pooled"]
    assert before > 0.03 and after < 0.5 * before


def test_unobserved_position_keeps_identity():
    z, n, _ = calibration_trace(61, 200, 3, 1.5)
    o = np.minimum(np.full(200, 2, np.int32), 2)
    r = oracle.sts_fit(z, np.minimum(n, 2), observed_len=o, grid=129)
    assert r["T"][2] == 1.0 and r["n_obs"][2] == 0
