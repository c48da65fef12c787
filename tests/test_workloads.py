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


def test_draft_overlap_tracks_confidence():
    """Each draft row's noise is chosen so that its acceptance probability, the overlap
    sum_v min(p_t, p_d) of the oracle's label, is the request's drawn confidence."""
    from oracle.acceptance import softmax64, tv_label

    inp = Inputs(get("mixed-b64"))
    for b in range(3):
        tl, dl, _ = inp.request_logits(b)
        t, d = tl.double().numpy(), dl.double().numpy()
        c = inp.conf64(b)
        for k in range(inp.wl.G1):
            ov = tv_label(softmax64(d[k]), softmax64(t[k]))
            assert abs(ov - c[k]) < 0.03, (b, k, ov, c[k])


def test_head_hidden_uses_the_drawn_confidence():
    """The head workload's hidden states encode the same confidences that set its draft
    noise: the head's logit on the (unrounded) hidden state is log(c / (1 - c))."""
    inp = Inputs(get("qwen3-4b"))
    h = inp.hidden().double().numpy()
    w = inp.head_w.astype(np.float64)
    for b in range(2):
        c = inp.conf64(b)
        z = h[b] @ w + float(inp.head_b)
        np.testing.assert_allclose(1.0 / (1.0 + np.exp(-z)), c, atol=2e-2)
