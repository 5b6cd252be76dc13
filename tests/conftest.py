import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs; minutes of CPU or GPU time")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built library on a GPU; fails loudly (never skips to a fallback) when absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import scaled_dot_product_sdpa_amd as sdpa
    sdpa.load()  # raises if libsdpa.so is missing
    return sdpa
