"""GPU parity of rva_markov_sample (Markov sequential head) against the oracle.

Bar: stored logits bit-exact (the int8 dot is exact and the float64 logit uses the same
rounded operations on both sides); drawn tokens bit-exact except a draw whose oracle margin
to a bin edge is below 1e-9 of the total mass (then that request's later positions, which
depend on the token, are left out and counted); probability of the drawn token <= 1e-12
relative.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ragged_verify_acceptance_amd import rva
from workloads.generate import markov_inputs

pytestmark = pytest.mark.gpu

DRAW_BAND = 1e-9


def _run(inp, B, G1, V, r):
    dev = "cuda"
    U = inp["U"].to(dev)
    out = torch.empty_like(U)
    tokens = torch.empty((B, G1), dtype=torch.int32, device=dev)
    p_at = torch.empty((B, G1), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(rva.markov_workspace_size(B, V), dtype=torch.uint8, device=dev)
    t = lambda x, d: torch.as_tensor(np.ascontiguousarray(x)).to(d).to(dev)
    rva.markov_sample(B, G1, V, r, U, t(inp["anchor"], torch.int32), t(inp["u"], torch.float32),
                      t(inp["q1"], torch.int8), t(inp["s1"], torch.float32), t(inp["q2"], torch.int8),
                      t(inp["s2"], torch.float32), out, tokens, p_at, ws, status)
    torch.cuda.synchronize()
    return out.cpu(), tokens.cpu().numpy(), p_at.cpu().numpy(), int(status.item())


def _compare(inp, reqs, out, tokens, p_at):
    sub = {k: (v[reqs] if k in ("U", "anchor", "u") else v) for k, v in inp.items()}
    ref = oracle.markov_sample(sub["U"], sub["anchor"], sub["u"], inp["q1"], inp["s1"], inp["q2"],
                               inp["s2"])
    flipped = 0
    for j, b in enumerate(reqs):
        for k in range(tokens.shape[1]):
            assert torch.equal(out[b, k].view(torch.int16) if out.dtype == torch.bfloat16 else out[b, k].view(torch.int32),
                               ref["logits"][j, k].view(torch.int16) if out.dtype == torch.bfloat16 else ref["logits"][j, k].view(torch.int32)), (b, k)
            if ref["margins"][j, k] < DRAW_BAND:
                flipped += 1
                break  # later positions depend on this draw
            assert tokens[b, k] == ref["tokens"][j, k], (b, k, tokens[b, k], ref["tokens"][j, k])
            assert abs(p_at[b, k] - ref["p_at"][j, k]) <= 1e-6 * ref["p_at"][j, k] + 1e-30
    return flipped


CASES = [
    # name, B, G1, V, r, dtype, requests checked (None: all)
    ("small-f32", 5, 4, 1000, 64, "f32", None),
    ("small-bf16-r128", 3, 6, 4096, 128, "bf16", None),
    ("ragged-vocab", 70, 3, 1003, 256, "bf16", None),     # V not a multiple of 8, B > 64
    ("two-groups-vec", 80, 2, 4096, 256, "bf16", None),   # B > 64 on the 16-byte path
    ("mixed-b64", 64, 7, 151936, 256, "bf16", [0, 17, 40, 63]),
    ("one-request-one-draft", 1, 1, 333, 128, "bf16", None),  # B = 1, G1 = 1, V < 3 tiles
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_markov_matches_oracle(case):
    name, B, G1, V, r, dtype, reqs = case
    print(f"[markov] {name} B={B} G1={G1} V={V} r={r} {dtype}", flush=True)
    inp = markov_inputs(300 + [c[0] for c in CASES].index(name), B, G1, V, r=r, dtype=dtype)
    out, tokens, p_at, status = _run(inp, B, G1, V, r)
    assert status == 0
    flipped = _compare(inp, list(range(B)) if reqs is None else reqs, out, tokens, p_at)
    print(f"[markov] {name}: draws inside the flip band: {flipped}", flush=True)
    assert flipped <= 1


def test_markov_bad_anchor_flags():
    inp = markov_inputs(9, 2, 2, 512, r=64, dtype="f32")
    inp["anchor"] = np.array([3, 600], np.int32)
    _, tokens, _, status = _run(inp, 2, 2, 512, 64)
    assert status & rva.DEV_BAD_TOKEN
    assert np.all((tokens >= 0) & (tokens < 512))
