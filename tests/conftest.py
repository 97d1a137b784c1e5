import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding; GPU tests only."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_moe_ffn_amd as F

    F.load()  # raises if the shared library was not built
    return F
