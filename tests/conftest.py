import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C ABI")
    config.addinivalue_line(
        "markers", "slow: longer CPU test (still part of the default CPU suite)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests only."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from jl_rotated_bit_amd import qjl
    qjl.load()
    return qjl
