import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libsherry.so")


@pytest.fixture(scope="session")
def gpu_lib():
    """The ctypes binding over libsherry.so on cuda:0; GPU tests only."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from ultra_bit_weight_amd import sherry

    sherry.load()  # raises if the library is missing
    return sherry
