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
