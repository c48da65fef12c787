import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where no GPU is visible, so that
    # ``pytest -m "not gpu"`` and plain ``pytest`` both work on a CPU-only host.
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build librva.so once if it is missing (hipcc cross-compiles without a GPU)."""
    from ragged_verify_acceptance_amd import build as _build

    if not os.path.exists(_build.LIB_PATH):
        _build.build(verbose=True)
    yield


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Flip counts of the GPU parity tests: requests whose integer outputs differ from the
    oracle inside the flip band (accept test |u - p_t/p_d| < 1e-6, draw u*S within 1e-9*S of
    a bin edge, scheduler near-tie), per test."""
    try:
        from tests.reference import FLIPS
    except Exception:  # pragma: no cover
        return
    if not FLIPS:
        return
    tw = terminalreporter
    total_c = sum(c for c, _ in FLIPS.values())
    total_f = sum(f for _, f in FLIPS.values())
    tw.write_sep("-", f"flip counts: {total_f} in band over {total_c} checked decisions/requests")
    for tag, (c, f) in sorted(FLIPS.items()):
        tw.write_line(f"  {tag}: {f} / {c}")
