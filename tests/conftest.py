import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Name each GPU test on stdout before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
