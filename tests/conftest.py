import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: oracle-heavy case (tens of seconds of CPU)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def psi_lib():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from memory_bounded_weight_amd import psi
    return psi
