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
    config.addinivalue_line("markers", "slow: long-running (large workloads)")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    """Write the test id to the real stderr before a GPU test runs, so a run
    that dies inside a kernel still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-test] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
