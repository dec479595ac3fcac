import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "memory: peak-memory test, run in a fresh subprocess")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture
def rng():
    """A fresh seeded generator per test, so no test depends on test order."""
    import numpy as np

    return np.random.default_rng(12345)
