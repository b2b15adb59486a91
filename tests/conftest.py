import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library through its C ABI)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def O():
    """The CPU oracle module (built on first use)."""
    from oracle import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def O_lib(O):
    """Oracle plus the HIP library; a missing library is an error, not a skip."""
    from microscaling_fp4_block_fp4q_amd import fp4q
    fp4q.lib()
    return O
