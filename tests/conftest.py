import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


@pytest.fixture(scope="session")
def gpu():
    """cuda:0 with libfa loaded.  Skips only when there is no GPU at all; a
    missing or broken library on a GPU machine is an error, not a skip."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from exact_attention_70_amd import binding
    binding.load_library()
    return torch.device("cuda:0")


def max_abs(a, b):
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
