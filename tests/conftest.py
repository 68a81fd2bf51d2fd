import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def max_rel_err(x, ref):
    """Normwise max relative error: ||x - ref||_inf / ||ref||_inf."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0:
        return float(num)
    return float(num / den)


@pytest.fixture
def rel_err():
    return max_rel_err
