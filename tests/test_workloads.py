"""CPU checks of the seeded input generator (determinism, independence, shapes) and of the
stored high-concurrency cost slope."""

import importlib.util
import os

import numpy as np

from workloads import Inputs, WORKLOADS, get
from workloads.configs import THETA_HIGH_CONCURRENCY

HERE = os.path.dirname(os.path.abspath(__file__))


def test_deterministic_and_per_request():
    wl = get("tiny")
    a, b = Inputs(wl), Inputs(wl)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_table, b.block_table)
    ta, da, xa = a.request_logits(2)
    tb, db, xb = b.request_logits(2)
    assert (ta == tb).all() and (da == db).all() and np.array_equal(xa, xb)
    # request 2 does not depend on having generated requests 0, 1 first
    c = Inputs(wl)
    q1 = c.request_qkv(2)[0]
    assert (q1 == a.request_qkv(2)[0]).all()


def test_page_table_is_a_permutation():
    for name in ("tiny", "mixed-b64"):
        inp = Inputs(get(name))
        used = np.concatenate([inp.block_table[b, : inp.pages_per_req[b]] for b in range(inp.B)])
        assert sorted(used.tolist()) == list(range(inp.num_pages))
        for b in range(inp.B):
            assert inp.pages_per_req[b] * inp.wl.page >= inp.context_lens[b] + inp.wl.gamma


def test_shapes():
    for wl in WORKLOADS.values():
        assert wl.tiers[-1] >= wl.B * wl.gamma
        assert wl.Hq % wl.Hkv == 0


def test_theta_high_concurrency_is_current():
    spec = importlib.util.spec_from_file_location("mk", os.path.join(HERE, "golden", "make_theta_high_concurrency.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    theta, mean_w = mk.derive()
    assert theta == THETA_HIGH_CONCURRENCY
    assert mean_w == 3.0
