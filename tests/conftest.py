import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than ~10 s on the CPU")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name the case on stdout (flushed) before a GPU test touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
