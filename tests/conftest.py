import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, where a GPU is visible. Fails (never skips) if the library is missing."""
    if not _gpu_present():
        pytest.skip("no GPU visible to torch")
    import exact_attention_45_amd as mi
    mi.load()  # raises if the shared library is missing or broken
    return mi
