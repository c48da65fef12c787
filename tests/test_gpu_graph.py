"""GPU: the verify step captured as one HIP graph, and the step-cost table measured with it.

* Replays of the captured step (schedule -> pack -> attention -> accept + labels) are
  bit-identical to the eager step, replay after replay, with eager steps and host
  synchronisation in between; a second batch of confidences (other windows, another tier)
  replays through the same graph and again matches its own eager step.
* The cost grid T(bs, M) measured by graph replay fits the additive model, and the
  scheduling call on the fitted (tier-aware) tables picks the oracle's windows.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ragged_verify_acceptance_amd.costmodel import fit_additive, scheduler_tables, tier_of
from ragged_verify_acceptance_amd.graph import CallGraph
from tests.reference import oracle_conf, to_np
from workloads import Inputs, get
from workloads.costgrid import measure
from workloads.device import DeviceStep

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits, so NaN labels and float outputs compare exactly."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    elif t.dtype == torch.float64:
        t = t.view(torch.int64)
    return t.cpu().numpy().copy()


def _snapshot(ds: DeviceStep) -> dict:
    torch.cuda.synchronize()
    M, tier = (int(x) for x in ds.total_tier.cpu())
    return {"windows": _bits(ds.windows), "K": _bits(ds.K_out), "ratio": _bits(ds.ratio_out),
            "conf": _bits(ds.conf_out), "surv": _bits(ds.surv_out), "cu": _bits(ds.cu),
            "total_tier": _bits(ds.total_tier), "row_req": _bits(ds.row_req[:tier]),
            "row_pos": _bits(ds.row_pos[:tier]), "pack_dst": _bits(ds.pack_dst[:tier]),
            "out": _bits(ds.out[:tier]), "accept_len": _bits(ds.accept_len),
            "committed": _bits(ds.committed), "context_lens": _bits(ds.context_lens),
            "labels": _bits(ds.labels), "pt_at": _bits(ds.pt_at), "pd_at": _bits(ds.pd_at),
            "status": _bits(ds.status)}


def _same(a: dict, b: dict, what: str):
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.parametrize("name", ["tiny", "qwen3-4b"])
def test_graph_replays_match_eager(name):
    print(f"[graph] {name}", flush=True)
    inp = Inputs(get(name))
    ds = DeviceStep(inp)
    ds.prepare()
    ds.restore()
    ds.step()
    ref = _snapshot(ds)
    assert int(ref["status"][0]) == 0

    ds.restore()
    g = CallGraph(ds.step)
    for rep in range(3):
        ds.restore()
        g.replay()
        _same(ref, _snapshot(ds), f"replay {rep}")
        ds.restore()
        ds.step()                       # eager work between replays
        _same(ref, _snapshot(ds), f"eager after replay {rep}")

    # new confidences -> other windows and (here) another tier, same graph
    if ds.conf_in is not None:
        ds.conf_in.copy_(ds.conf_in ** 6)
    else:
        ds.head_w.mul_(-1.0)            # flips every head logit: low confidences
    ds.restore()
    ds.step()
    ref2 = _snapshot(ds)
    t1, t2 = int(ref["total_tier"][1]), int(ref2["total_tier"][1])
    print(f"[graph] {name} tier {t1} -> {t2}", flush=True)
    assert t2 < t1
    for rep in range(2):
        ds.restore()
        g.replay()
        _same(ref2, _snapshot(ds), f"replay at the second tier {rep}")


def test_cost_grid_fit_and_scheduler_on_measured_tables():
    name = "qwen3-4b"
    print(f"[costgrid] {name}", flush=True)
    inp = Inputs(get(name))
    wl = inp.wl
    ds = DeviceStep(inp)
    ds.prepare()
    samples, sched = measure(ds, [1, 2, 4, 8, 16], reps=7, warm=2)
    assert len(samples) > 20 and all(t > 0 for _, _, t in samples)
    f = fit_additive(samples, ds.tiers)
    print(f"[costgrid] rms {f.rms:.2f} us, alpha {np.round(f.alpha, 1)}, "
          f"theta(top) {f.theta[-1]:.1f} us, schedule {sched}", flush=True)
    assert np.all(np.isfinite(f.alpha)) and np.all(np.isfinite(f.theta))
    T = {(b, m): t for b, m, t in samples}
    # more requests and more rows cost more; the additive model explains the grid
    assert T[(16, 96)] > T[(1, 1)]
    assert f.rms < 0.25 * float(np.mean([t for _, _, t in samples]))

    # the scheduler consumes the measured, tier-aware tables (microseconds -> ms)
    bias, alpha, theta = scheduler_tables(f, inp.B, wl.gamma, ds.tiers)
    alpha_ms, theta_ms = (alpha * 1e-3).astype(np.float32), (theta * 1e-3).astype(np.float32)
    ds.bias = float(bias)
    ds.alpha = torch.from_numpy(alpha_ms).cuda()
    ds.theta = torch.from_numpy(theta_ms).cuda()
    ds.schedule()
    torch.cuda.synchronize()
    a = oracle.survival(oracle_conf(inp))
    r = oracle.schedule_windows(a, wl.gamma, np.float32(bias), alpha_ms, theta_ms)
    if not r["near_tie"]:
        assert np.array_equal(to_np(ds.windows), r["windows"])
        assert int(ds.K_out.item()) == r["K"]
    M = int(np.sum(r["windows"]))
    assert M == inp.B * wl.gamma or M == tier_of(M, ds.tiers) or r["near_tie"]
