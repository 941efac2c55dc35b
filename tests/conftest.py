import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# the two forward kernels an unsplit call can run, forced by name
FWD_KERNELS = ["pipelined", "pingpong"]


@pytest.fixture(params=FWD_KERNELS)
def fwd_kernel(request, monkeypatch):
    """Force one forward kernel for the test (the library reads FLASH_ATTN_FWD_KERNEL
    at every call)."""
    monkeypatch.setenv("FLASH_ATTN_FWD_KERNEL", request.param)
    return request.param
