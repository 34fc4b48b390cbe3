import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the C oracle once if it is missing (it is test infrastructure)."""
    from oracle import runner
    if not os.path.exists(runner.library_path()):
        runner.build(force=False)
    yield
