import os
import sys

import pytest

# Load PyTorch (and its HIP runtime) before anything loads libtopk.so, so that
# the process holds exactly one HIP runtime.
import torch  # noqa: F401,E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
