"""Sequential Temperature Scaling (fitting) and expected calibration error.

TEST INFRASTRUCTURE (part of the CPU oracle package; see ``oracle/__init__.py``).

Sources:

* [NOTES] section 07 ("为什么还要做 Sequential Temperature Scaling？"): the head's scores
  are over-confident; a temperature per draft position is fitted so that the prefix
  survival it predicts matches the rate at which prefixes actually survive verification.
* [SGL] "DSpark：sequential head 加验证预算": STS calibrates the block's survival to the
  real acceptance rate.
* [CSDN] section 5 ("可观测性"): per-request confidence and calibration metrics such as
  ECE for after-the-fact analysis; only full-block (static, cap-accept) runs observe
  positions past the scheduled window.

Readings (the pages give no formula):

* A trace sample i holds the head logits ``z[i, k]`` of the gamma-1 draft positions, the
  number of drafts a full-block verification accepted, ``n_i`` (0 .. gamma-1), and the
  number of positions observed, ``o_i`` (gamma-1 for full-block runs; w_i - 1 for compact
  runs, whose later positions were never verified).  Position k (1-based) is observed iff
  ``k <= o_i``; its outcome is ``E[i, k] = [n_i >= k]``: the prefix of length k survived.
* With temperatures T, the predicted prefix survival is
  ``a[i, k] = prod_{j <= k} sigmoid(z[i, j] / T_j)``, formed as exp of a float64 sum of
  log-sigmoids.
* "Sequential": T_1 is fitted first, then T_2 with T_1 fixed, and so on.  T_k minimises
  the Bernoulli negative log-likelihood of the observed E[., k] under a[., k] over
  ``T_k in [T_lo, T_hi]`` (the global minimum on that interval).  A position with no
  observed sample keeps T_k = 1.
* ECE: the observed (a, E) pairs are put in ``n_bins`` equal-width bins of a on [0, 1]
  (bin = min(floor(a * n_bins), n_bins - 1)); ECE = sum over bins of
  (count / total) * |mean a - mean E|.  Reported pooled over positions and per position.

Parity unpinned: that this is the fit the pages' authors ran (no page prints fitted
temperatures or an ECE value).  Pinned: the estimator's definition (a single position is
plain temperature scaling, i.e. logistic regression on z without intercept; recovery of
known temperatures on large synthetic traces; optimality), and ECE on hand examples and
closed forms.
"""

from __future__ import annotations

import numpy as np
from scipy.optimize import minimize_scalar
from scipy.special import log_expit


def _log1mexp(y):
    """log(1 - exp(y)) for y <= 0, accurate at both ends."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty_like(y)
    small = y > -np.log(2.0)
    out[small] = np.log(-np.expm1(y[small]))
    out[~small] = np.log1p(-np.exp(y[~small]))
    return out


def observed_outcomes(accept_len, observed_len, G1):
    """(observed [N, G1] bool, E [N, G1] bool) from accept lengths and observed lengths."""
    n = np.asarray(accept_len, dtype=np.int64)
    N = n.shape[0]
    o = np.full(N, G1, np.int64) if observed_len is None else np.asarray(observed_len, np.int64)
    k = np.arange(1, G1 + 1)[None, :]
    return (k <= o[:, None]), (n[:, None] >= k)


def log_prefix_survival(z, T):
    """float64 [N, G1]: log a[i, k] = sum_{j <= k} log sigmoid(z[i, j] / T_j), summed in
    position order."""
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    T = np.ones(z.shape[1]) if T is None else np.asarray(T, dtype=np.float32).astype(np.float64)
    N, G1 = z.shape
    L = np.empty((N, G1))
    acc = np.zeros(N)
    for k in range(G1):
        acc = acc + log_expit(z[:, k] / T[k])
        L[:, k] = acc
    return L


def position_nll(z_k, L_prev, E_k, obs_k, T):
    """Negative log-likelihood of position k's observed outcomes at temperature T, given the
    log survival of the earlier positions (already calibrated)."""
    la = L_prev[obs_k] + log_expit(np.float64(z_k[obs_k]) / T)
    e = E_k[obs_k]
    return float(-(np.sum(la[e]) + np.sum(_log1mexp(la[~e]))))


def sts_fit(z, accept_len, observed_len=None, T_lo=0.05, T_hi=20.0, grid=4097):
    """Sequential temperature fit.  Returns dict(T float32 [G1], T64 float64 [G1],
    nll float64 [G1], n_obs int [G1], near_tie bool [G1]).

    The minimum over [T_lo, T_hi] is located on a ``grid``-point log-spaced scan and refined
    by a bounded scalar minimisation inside the neighbouring grid cells; ``near_tie`` flags
    a second grid point, outside those cells, within 1e-9 (relative) of the best value
    (two basins: a fit there is not unique)."""
    z = np.asarray(z, dtype=np.float32)
    N, G1 = z.shape
    obs, E = observed_outcomes(accept_len, observed_len, G1)
    # the bracket ends are float32 values (as a caller passes them to the library)
    T_lo, T_hi = float(np.float32(T_lo)), float(np.float32(T_hi))
    u = np.linspace(np.log(T_lo), np.log(T_hi), grid)
    T_fit = np.ones(G1)
    nll = np.zeros(G1)
    near = np.zeros(G1, bool)
    L_prev = np.zeros(N)
    zd = z.astype(np.float64)
    for k in range(G1):
        if obs[:, k].any():
            f = np.array([position_nll(zd[:, k], L_prev, E[:, k], obs[:, k], np.exp(x)) for x in u])
            j = int(np.argmin(f))
            lo, hi = u[max(j - 1, 0)], u[min(j + 1, grid - 1)]
            r = minimize_scalar(lambda x: position_nll(zd[:, k], L_prev, E[:, k], obs[:, k], np.exp(x)),
                                bounds=(lo, hi), method="bounded", options={"xatol": 1e-12})
            x = r.x if r.fun <= f[j] else u[j]
            T_fit[k] = np.exp(x)
            nll[k] = position_nll(zd[:, k], L_prev, E[:, k], obs[:, k], T_fit[k])
            far = np.abs(np.arange(grid) - j) > 1
            near[k] = bool(np.any(f[far] <= f[j] * (1 + 1e-9) + 1e-300))
        L_prev = L_prev + log_expit(zd[:, k] / T_fit[k])
    return {"T": T_fit.astype(np.float32), "T64": T_fit, "nll": nll,
            "n_obs": obs.sum(axis=0), "near_tie": near}


def ece(z, accept_len, observed_len=None, T=None, n_bins=15):
    """Expected calibration error of the predicted prefix survival.

    Returns dict(pooled float64, per_position float64 [G1], counts int [G1, n_bins],
    sum_a float64 [G1, n_bins], sum_e int [G1, n_bins], boundary int): ``boundary`` counts
    observed pairs whose a * n_bins lies within 1e-9 of a bin edge (a binning that another
    rounding of a may flip)."""
    z = np.asarray(z, dtype=np.float32)
    N, G1 = z.shape
    obs, E = observed_outcomes(accept_len, observed_len, G1)
    a = np.exp(log_prefix_survival(z, T))
    counts = np.zeros((G1, n_bins), np.int64)
    sum_a = np.zeros((G1, n_bins))
    sum_e = np.zeros((G1, n_bins), np.int64)
    boundary = 0
    for i in range(N):
        for k in range(G1):
            if not obs[i, k]:
                continue
            x = a[i, k] * n_bins
            b = min(int(np.floor(x)), n_bins - 1)
            if abs(x - round(x)) < 1e-9 and 0 < round(x) < n_bins:
                boundary += 1
            counts[k, b] += 1
            sum_a[k, b] += a[i, k]
            sum_e[k, b] += int(E[i, k])

    def _ece(c, sa, se):
        tot = c.sum()
        if tot == 0:
            return 0.0
        m = c > 0
        return float(np.sum(c[m] / tot * np.abs(sa[m] / c[m] - se[m] / c[m])))

    per = np.array([_ece(counts[k], sum_a[k], sum_e[k]) for k in range(G1)])
    pooled = _ece(counts.sum(0), sum_a.sum(0), sum_e.sum(0))
    return {"pooled": pooled, "per_position": per, "counts": counts, "sum_a": sum_a,
            "sum_e": sum_e, "boundary": boundary}
