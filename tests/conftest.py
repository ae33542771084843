import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def gpu_visible() -> bool:
    """True when a GPU may be reachable from this process. CPU tests that hand
    fake device addresses to an entry point whose validation they expect to
    pass would launch a kernel on those addresses there, so they skip.
    (torch.cuda.device_count() does not initialise the HIP runtime.)"""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


GPU_VISIBLE = gpu_visible()
no_gpu_only = pytest.mark.skipif(
    GPU_VISIBLE, reason="passes validation with fake device pointers: would launch a kernel on a GPU")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle
