import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lq():
    """The HIP binding, loaded once; GPU tests fail (not skip) if it is missing."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from bit_ptq_looped_amd import loopq
    loopq.load()
    return loopq
