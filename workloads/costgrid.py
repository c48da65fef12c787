"""Measures the verify step's cost T(bs, M) on the device by graph replay.

For each batch size bs (the first bs requests of a workload) one graph of the verify
calls (pack -> attention -> accept with labels) is captured and replayed with windows that
sum to each M on the grid; a second graph holds the scheduling call, whose cost does not
depend on M.  Times are the median of HIP-event intervals around single replays on the
launch stream; context_lens is restored between replays, outside the intervals.

Harness code: drives the binding and records times; the fit lives in
``ragged_verify_acceptance_amd.costmodel``.
"""

from __future__ import annotations

import numpy as np
import torch

from ragged_verify_acceptance_amd.costmodel import even_windows
from ragged_verify_acceptance_amd.graph import CallGraph

from .device import DeviceStep, prepare_with_windows


def grid_points(bs: int, gamma: int, tiers) -> list:
    """M values for one bs: bs itself, every tier in (bs, bs*gamma], and bs*gamma."""
    top = bs * gamma
    ms = {bs, top} | {int(t) for t in tiers if bs < t <= top}
    return sorted(ms)


def time_replays(graph: CallGraph, before, reps: int, warm: int) -> float:
    """Median microseconds of one replay (HIP events on the current stream)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        if before is not None:
            before()
        graph.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        if before is not None:
            before()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3)


def measure(ds: DeviceStep, bs_list, reps: int = 20, warm: int = 3, labels: bool = True):
    """Returns (samples [(bs, M, T_us)], schedule_us {bs: T_us}); ds.B is restored after."""
    wl = ds.wl
    B0 = ds.B
    samples, sched = [], {}
    try:
        for bs in bs_list:
            if not 1 <= bs <= B0:
                raise ValueError(f"bs={bs} outside [1, {B0}]")
            ds.B = bs
            pts = grid_points(bs, wl.gamma, ds.tiers)
            prepare_with_windows(ds, even_windows(bs, pts[-1], wl.gamma))
            ds.restore()

            def verify():
                ds.pack()
                ds.attention()
                ds.accept(labels=labels)

            g = CallGraph(verify)
            for M in pts:
                prepare_with_windows(ds, even_windows(bs, M, wl.gamma))
                samples.append((bs, M, time_replays(g, ds.restore, reps, warm)))
            del g
            gs = CallGraph(ds.schedule)
            sched[bs] = time_replays(gs, None, reps, warm)
            del gs
    finally:
        ds.B = B0
        ds.restore()
    return samples, sched
