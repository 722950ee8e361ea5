import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    return o


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gq():
    """The GPU library binding; GPU tests fail loudly if it is not built."""
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import gguf_block_quant_gq_amd as g
    g.load_library()  # raises if libgq.so is missing
    return g
