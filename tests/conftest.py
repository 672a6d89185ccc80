import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; on a host without one they are skipped
    # rather than failed, so that `-m "not gpu"` and plain runs behave.
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


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    # Name each GPU test on the real stderr before it runs, so that a run that
    # ends abruptly still shows which case was on the device.
    if "gpu" in request.node.keywords:
        sys.__stderr__.write(f"\n[gpu test] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
