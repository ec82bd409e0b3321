import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _guard_canaries(request):
    """After every GPU test: the canaries around each buffer the test took
    from gpu_util.G must be intact (no kernel stored outside its outputs)."""
    yield
    if request.node.get_closest_marker("gpu") is not None and "gpu_util" in sys.modules:
        sys.modules["gpu_util"].G.check()
