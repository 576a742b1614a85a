import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running full-size case")


def gpu_available() -> bool:
    """True when a GPU is visible. Counting devices does not initialise HIP."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (fails loudly if it
    has not been built)."""
    from fp8_quantised_paged_amd import kvfp8
    return kvfp8
