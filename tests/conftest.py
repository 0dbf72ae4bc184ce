import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with the HIP library loaded (a missing library is an error, not a skip)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_attention_amd as mla
    mla.lib()
    return torch.device("cuda:0")
