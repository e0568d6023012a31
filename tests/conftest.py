import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive CPU checks (tens of seconds)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.get()


@pytest.fixture(scope="session")
def native_dir(tmp_path_factory):
    """Compiled test-side native checkers (built once per session)."""
    return tmp_path_factory.mktemp("native")
