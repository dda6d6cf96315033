import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


@pytest.fixture(scope="session")
def lib():
    """The HIP C-ABI library through its Python binding (fails loudly if unbuilt)."""
    import w8a16_linear_layers_amd as fp8lin

    return fp8lin.load_library()


@pytest.fixture(scope="session")
def gpu():
    """Skips nothing: a GPU test run without a GPU is an error, not a skip."""
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU test selected but torch.cuda.is_available() is False")
    return torch.device("cuda", 0)
