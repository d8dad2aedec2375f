import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case")


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run before touching the device, so a
    # crash report names it; nothing to reorder here.
    pass


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on the real stderr before it touches the device, so
    that a run that ends abruptly still says which case was running."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
