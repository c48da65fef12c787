"""rva_verify_attention_noalloc against rva_verify_attention, through the C ABI.

The no-workspace variant runs the same kernels with the library's static scratch in place
of the caller's workspace, so its output must be bit-identical to the workspace variant's
on the same inputs (the bar for attention against the oracle is 1e-2 relative; identical
kernels on identical inputs give identical bits).  Two calls in a row: the mixed-traffic
batch (B = 64, contexts up to 8K), then a smaller batch (B = 16 of the same workload), so
the second call reuses scratch the first one left behind.  The appended window K/V must be
the same as well, and one request of each call is also checked against the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from ragged_verify_acceptance_amd import rva
from tests.reference import attn_rel_err, oracle_attention, oracle_schedule
from workloads import Inputs, get
from workloads.device import DeviceStep, prepare_with_windows

pytestmark = pytest.mark.gpu


def _noalloc(ds):
    wl, inp = ds.wl, ds.inp
    rva.verify_attention_noalloc(ds.B, wl.gamma, ds.max_rows, wl.Hq, wl.Hkv, wl.D, wl.page,
                                 inp.num_pages, inp.max_pages, ds.q, ds.k_new, ds.v_new,
                                 ds.k_cache, ds.v_cache, ds.block_table, ds.context_lens, ds.cu,
                                 ds.total_tier, ds.scale, ds.out, ds.status)


@pytest.mark.parametrize("B", [64, 16], ids=["B64-first", "B16-second"])
def test_noalloc_matches_workspace_variant(B):
    print(f"[noalloc] mixed-b64 B={B}", flush=True)
    inp = Inputs(get("mixed-b64"), B=B)
    ds = DeviceStep(inp)
    windows = oracle_schedule(inp)["windows"]
    prepare_with_windows(ds, windows)
    need = rva.verify_attention_workspace_size(B, ds.wl.gamma, ds.wl.Hq, ds.wl.Hkv, ds.wl.D,
                                               ds.wl.page, inp.max_pages, rva.BF16)
    assert 0 < need <= 24 << 20
    ds.status.zero_()
    ds.out.fill_(3.0)
    ds.attention()
    torch.cuda.synchronize()
    ref_out = ds.out.clone()
    ref_k, ref_v = ds.k_cache.clone(), ds.v_cache.clone()
    tier = int(ds.total_tier[1].item())
    for rep in range(2):  # twice: the second call starts from the scratch the first left
        ds.out.fill_(3.0)  # the same fill as the reference call: rows past the tier keep it
        _noalloc(ds)
        torch.cuda.synchronize()
        assert int(ds.status.item()) == 0
        assert torch.equal(ds.out.view(torch.int16), ref_out.view(torch.int16)), f"call {rep}: output differs"
        assert bool(torch.all(ds.out[tier:] == 3.0))
        assert torch.equal(ds.k_cache.view(torch.int16), ref_k.view(torch.int16))
        assert torch.equal(ds.v_cache.view(torch.int16), ref_v.view(torch.int16))
    b = B - 1
    ref, _, _ = oracle_attention(inp, windows, [b])
    cu = ds.cu.cpu().numpy()
    err = attn_rel_err(ds.out.float().cpu().numpy()[cu[b]:cu[b + 1]], ref[b])
    assert err <= 1e-2, err
    del ds
    torch.cuda.empty_cache()
