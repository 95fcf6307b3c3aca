import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (built once if absent; never a fallback)."""
    from linear_attention_recurrent_amd import binding
    if not os.path.exists(binding.library_path()):
        from linear_attention_recurrent_amd import build as _build
        _build.build()
    return binding.load_library()


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU (run with -m 'not gpu' here)")
    return torch.device("cuda:0")
