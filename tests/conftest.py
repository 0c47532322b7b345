import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_sync_after_test(request):
    """For GPU tests: name the test before it touches the device, and synchronise after it so
    that an asynchronous device error is attributed to the test that caused it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    print(f"\n>>> {request.node.nodeid}", flush=True)
    yield
    import torch
    if torch.cuda.is_available():
        torch.cuda.synchronize()
