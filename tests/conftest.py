import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def based():
    """The HIP binding, on a machine with a GPU.  Fails (never skips) when the
    GPU is there but the library is not: the GPU tests must run native code."""
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import linear_attention_lm_amd as lal

    return lal
