import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--seer-lib", default=None,
                     help="path of the libseer build the tests load (default: the in-tree one)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib(request):
    """The built C-ABI library (never the oracle)."""
    from block_sparse_attention_29_amd import seer
    path = request.config.getoption("--seer-lib")
    return seer.load(path) if path else seer.load()
