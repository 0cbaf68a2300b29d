import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def wkv():
    """The HIP library binding on cuda:0 (GPU tests only; fails loudly without a GPU)."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    import rwkv_linear_attention_forward_amd as m
    return m


@pytest.fixture(scope="session")
def dev():
    import torch
    return torch.device("cuda:0")
