import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    # name the case before it touches the GPU, so a lost run still says which
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n>>> {request.node.nodeid}", flush=True)
    yield
