import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it touches the device, so a run
    that loses the GPU still shows which case was running."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield


@pytest.fixture
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    return torch.device("cuda:0")
