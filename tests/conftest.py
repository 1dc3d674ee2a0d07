import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (full-size oracle runs)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path through its C-ABI; fails loudly if the library is absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    from vision_transformer_sparse_amd import bra
    bra.load()
    return bra
