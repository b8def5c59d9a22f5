import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip (not fail) GPU tests on a machine without a GPU; fail loudly when
    a GPU is present but the HIP library is missing."""
    if not _gpu_available():
        pytest.skip("no GPU on this machine")
    import exact_attention_forward_attn_amd as ea
    ea.load()  # raises if the library is not built
    return ea
