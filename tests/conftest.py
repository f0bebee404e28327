import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The oracle is plain C; compile it once if no build is present."""
    from oracle import build_oracle
    if not os.path.exists(build_oracle.LIB):
        build_oracle.build()
    yield
