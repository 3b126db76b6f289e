import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


@pytest.fixture(autouse=True)
def _reset_oracle_fault():
    """Every test starts and ends with no planted fault in the oracle and the
    unclamped SiLU."""
    import oracle
    oracle.set_fault("none")
    oracle.set_activation_limit(0.0)
    yield
    oracle.set_fault("none")
    oracle.set_activation_limit(0.0)
