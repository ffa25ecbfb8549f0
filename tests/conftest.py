import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(autouse=True)
def _workspace_status(request):
    """GPU tests: every workspace's status word is still 0 after the test."""
    yield
    if request.node.get_closest_marker("gpu") is not None:
        from gpu_util import check_workspaces
        check_workspaces()
