import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly if it is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    from transformer_attention_sdpa_amd import _lib

    _lib.load()  # raises if the built library is absent
    return _lib
