import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running parity case at full workload size")


def to_np(inp):
    """Torch tensors (any dtype, any device) -> float64 numpy, losslessly."""
    out = {}
    for k, v in inp.items():
        out[k] = v.detach().to("cpu").to(dtype=__import__("torch").float64).numpy()
    return out


@pytest.fixture
def rng():
    return np.random.default_rng(12345)
