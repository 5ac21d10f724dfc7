import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with libeagle.so loaded; fails (not skips) if either is missing."""
    import torch
    from speculative_decoding_parent_amd import _lib
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    _lib.lib()
    return torch.device("cuda:0")
