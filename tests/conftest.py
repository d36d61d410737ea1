import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the oracle once if it is missing (gcc is available wherever the tests run)."""
    from oracle import build_oracle, oracle
    if not os.path.exists(oracle.LIB_PATH):
        build_oracle.build()
    yield
