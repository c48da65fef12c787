"""GPU: the step with the scheduling call overlapped on a second stream gives the same
outputs as the serial step (the confidences do not change between steps here, so the
windows scheduled one step ahead are the current step's)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from workloads import Inputs, get
from workloads.device import DeviceStep

pytestmark = pytest.mark.gpu


def _outs(ds):
    torch.cuda.synchronize()
    M, tier = (int(x) for x in ds.total_tier.cpu())
    return [ds.windows.cpu().numpy().copy(), ds.cu.cpu().numpy().copy(),
            ds.out[:tier].view(torch.int16).cpu().numpy().copy(),
            ds.accept_len.cpu().numpy().copy(), ds.committed.cpu().numpy().copy(),
            ds.context_lens.cpu().numpy().copy(), ds.labels.view(torch.int32).cpu().numpy().copy()]


@pytest.mark.parametrize("name", ["qwen3-4b", "mixed-b64"])
def test_overlapped_schedule_matches_serial(name):
    print(f"[overlap] {name}", flush=True)
    ds = DeviceStep(Inputs(get(name)))
    ds.prepare()
    ds.restore()
    ds.step()
    ref = _outs(ds)
    side = torch.cuda.Stream()
    ea, es = torch.cuda.Event(), torch.cuda.Event()
    for rep in range(4):
        ds.restore()
        ds.step_overlapped(side, ea, es)
        got = _outs(ds)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a, b), (rep, i)
    assert int(ds.status.item()) == 0
