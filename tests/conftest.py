import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def gpu():
    """Skip-free GPU guard: a gpu-marked test must find a GPU and the built
    library; a missing one is a failure, not a silent fallback."""
    import torch
    assert torch.cuda.is_available(), "gpu test run without a visible GPU"
    import int2_rotated_kv_write_amd as lib
    lib.load()
    return torch.device("cuda:0")
