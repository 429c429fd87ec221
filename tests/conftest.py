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
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU")


@pytest.fixture(scope="session")
def ora():
    import oracle
    return oracle.lib()


@pytest.fixture(autouse=True)
def _guard_bands(request):
    """GPU tests: every guarded device buffer (tests/gpu_util.py) keeps its
    canary bands intact through the test."""
    yield
    if request.node.get_closest_marker("gpu") is not None:
        import gpu_util
        gpu_util.GUARDS.check()
