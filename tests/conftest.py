import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload")


@pytest.fixture(scope="session")
def gpu():
    """Skip-free GPU fixture: a test marked gpu must have a device and the
    native library; anything else is an error, not a skip."""
    import torch
    assert torch.cuda.is_available(), "gpu-marked test run without a GPU"
    import sparse_kv_selection_amd as qk
    return qk
