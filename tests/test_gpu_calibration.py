"""GPU parity of the calibration calls (rva_sts_fit, rva_calibration_ece) against the oracle.

Inputs are synthetic acceptance traces from the seeded generator (known temperatures,
optional compact-mode censoring).  Bar:
* temperatures: |T_gpu / T_oracle - 1| <= 1e-5 (both locate the same minimum; the library's
  grid refinement ends at a spacing of ~1e-8 in ln T), unless the oracle flags two
  near-equal basins;
* minimised NLL per position: 1e-7 relative.  Position k's NLL is flat in T_k at the
  minimum but not in the earlier temperatures, so their differences (up to ~1e-8 in ln T
  each on either side) move it to first order: |dNLL / d ln T_j| is about N / 10, i.e.
  ~1e-6 absolute at N = 2000 over 15 positions;
* the library's T_k is a minimiser of the oracle's likelihood (with the oracle's earlier
  temperatures) to 1e-7 relative;
* ECE bin counts: bit-exact, except pairs the oracle finds within 1e-9 of a bin edge (a
  last-bit difference of the survival may move them one bin); ECE to 1e-9 plus those.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import log_expit

import oracle
from oracle.calibration import observed_outcomes, position_nll
from ragged_verify_acceptance_amd import rva
from workloads.generate import calibration_trace

pytestmark = pytest.mark.gpu

T_TOL = 1e-5
NLL_TOL = 1e-7


def _dev(x, dtype):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def _gpu_fit(z, n, o, T_lo=0.05, T_hi=20.0):
    N, G1 = z.shape
    T = torch.empty(G1, dtype=torch.float32, device="cuda")
    nll = torch.empty(G1, dtype=torch.float64, device="cuda")
    ws = torch.empty(rva.sts_fit_workspace_size(N), dtype=torch.uint8, device="cuda")
    rva.sts_fit(N, G1, _dev(z, torch.float32), _dev(n, torch.int32),
                None if o is None else _dev(o, torch.int32), T_lo, T_hi, T, nll, ws)
    torch.cuda.synchronize()
    return T.cpu().numpy(), nll.cpu().numpy()


def _gpu_ece(z, n, o, T, n_bins):
    N, G1 = z.shape
    out = torch.empty(G1 + 1, dtype=torch.float64, device="cuda")
    cnt = torch.empty((G1, n_bins), dtype=torch.int32, device="cuda")
    ws = torch.empty(rva.calibration_ece_workspace_size(N, G1, n_bins), dtype=torch.uint8,
                     device="cuda")
    rva.calibration_ece(N, G1, _dev(z, torch.float32), _dev(n, torch.int32),
                        None if o is None else _dev(o, torch.int32),
                        None if T is None else _dev(T, torch.float32), n_bins, out, cnt, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cnt.cpu().numpy()


CASES = [
    # name, N, G1, T_true, noise, censor, grid
    ("full-7", 3000, 7, [1.3, 1.5, 1.7, 1.9, 2.1, 2.3, 2.5], 0.3, False, 513),
    ("censored-5", 4000, 5, [1.4, 0.8, 2.0, 1.2, 1.6], 0.5, True, 513),
    ("one-position", 2500, 1, [1.7], 0.2, False, 1025),
    ("tiny-N", 5, 3, [1.5, 1.5, 1.5], 0.0, False, 513),
    ("large-N", 150000, 3, [1.2, 1.8, 2.4], 0.4, False, 129),
    ("gamma16", 2000, 15, 1.6, 0.3, False, 257),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sts_fit_matches_oracle(case):
    name, N, G1, T_true, noise, censor, grid = case
    print(f"[sts] {name} N={N} G1={G1}", flush=True)
    seed = 100 + [c[0] for c in CASES].index(name)
    z, n, o = calibration_trace(seed, N, G1, T_true, noise=noise, censor=censor)
    if censor:
        n = np.minimum(n, o)
    else:
        o = None
    ref = oracle.sts_fit(z, n, observed_len=o, grid=grid)
    T, nll = _gpu_fit(z, n, o)
    obs, E = observed_outcomes(n, o, G1)
    L = np.zeros(N)
    for k in range(G1):
        if ref["n_obs"][k] == 0:
            assert T[k] == 1.0 and nll[k] == 0.0
        elif not ref["near_tie"][k]:
            assert abs(T[k] / ref["T64"][k] - 1) <= T_TOL, (k, T[k], ref["T64"][k])
            assert abs(nll[k] - ref["nll"][k]) <= NLL_TOL * abs(ref["nll"][k]) + 1e-12
            # the library's temperature is (to rounding) a minimiser of the oracle's likelihood
            f_gpu = position_nll(z[:, k].astype(np.float64), L, E[:, k], obs[:, k], float(T[k]))
            assert f_gpu <= ref["nll"][k] * (1 + 1e-7) + 1e-12
        L = L + log_expit(z[:, k].astype(np.float64) / ref["T64"][k])


@pytest.mark.parametrize("n_bins", [15, 10, 64])
@pytest.mark.parametrize("calibrated", [False, True])
def test_ece_matches_oracle(n_bins, calibrated):
    G1 = 7 if n_bins < 64 else 5
    print(f"[ece] bins={n_bins} calibrated={calibrated}", flush=True)
    z, n, o = calibration_trace(77, 6000, G1, 1.8, noise=0.3, censor=True)
    n = np.minimum(n, o)
    T = oracle.sts_fit(z, n, observed_len=o, grid=257)["T"] if calibrated else None
    ref = oracle.ece(z, n, observed_len=o, T=T, n_bins=n_bins)
    out, cnt = _gpu_ece(z, n, o, T, n_bins)
    flips = int(np.abs(cnt - ref["counts"]).sum())
    assert flips <= 2 * ref["boundary"], (flips, ref["boundary"])
    tol = 1e-9 + 2.0 * ref["boundary"] / max(1, int(ref["counts"].sum()))
    assert abs(out[0] - ref["pooled"]) <= tol
    assert np.all(np.abs(out[1:] - ref["per_position"]) <= tol)


def test_ece_edges():
    """N = 1, a position nobody observed, and a confidence of exactly 1 (top bin)."""
    z = np.array([[40.0, -3.0, 0.5]], np.float32)
    n = np.array([1], np.int32)
    o = np.array([2], np.int32)
    ref = oracle.ece(z, n, observed_len=o, n_bins=10)
    out, cnt = _gpu_ece(z, n, o, None, 10)
    assert np.array_equal(cnt, ref["counts"])
    assert abs(out[0] - ref["pooled"]) < 1e-12 and out[3] == 0.0


def test_fit_then_ece_drops():
    """End to end on one trace: the fitted temperatures lower the ECE the library reports."""
    z, n, _ = calibration_trace(91, 20000, 7, 2.2, noise=0.3)
    T, _ = _gpu_fit(z, n, None)
    before, _ = _gpu_ece(z, n, None, None, 15)
    after, _ = _gpu_ece(z, n, None, T, 15)
    print(f"[ece] before {before[0]:.4f} after {after[0]:.4f}, T = {np.round(T, 3)}", flush=True)
    assert after[0] < 0.5 * before[0]


@pytest.mark.parametrize("kind", ["unobserved-tail", "all-survive"])
def test_sts_fit_degenerate(kind):
    """Positions nobody observed keep T = 1 with NLL 0; outcomes that are all survivals put
    the minimum on the bracket's lower end (sigmoid(z / T) -> 1 as T -> 0 for z > 0)."""
    print(f"[sts-degenerate] {kind}", flush=True)
    rng = np.random.default_rng(77)
    if kind == "unobserved-tail":
        N, G1 = 500, 5
        z = rng.normal(1.0, 1.5, size=(N, G1)).astype(np.float32)
        o = rng.integers(0, 3, size=N).astype(np.int32)  # positions 3..5 never observed
        n = np.minimum(rng.integers(0, G1 + 1, size=N), o).astype(np.int32)
    else:
        N, G1 = 300, 2
        z = rng.uniform(0.5, 3.0, size=(N, G1)).astype(np.float32)
        o = None
        n = np.full(N, G1, np.int32)
    ref = oracle.sts_fit(z, n, observed_len=o)
    T, nll = _gpu_fit(z, n, o)
    for k in range(G1):
        if ref["n_obs"][k] == 0:
            assert T[k] == 1.0 and nll[k] == 0.0
        else:
            assert abs(T[k] / ref["T64"][k] - 1) <= T_TOL, (k, T[k], ref["T64"][k])
            assert abs(nll[k] - ref["nll"][k]) <= NLL_TOL * abs(ref["nll"][k]) + 1e-12
    if kind == "unobserved-tail":
        assert list(ref["n_obs"][2:]) == [0, 0, 0]
    else:
        assert np.allclose(T, np.float32(0.05), rtol=1e-5)
