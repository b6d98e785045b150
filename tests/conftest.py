import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size parity case (minutes of oracle time)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; skips nothing -- a GPU test with no GPU or no
    library fails loudly."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test requested but no GPU is visible")
    import birkhoff_projection_amd as bp
    bp.lib()  # raises if the shared library is missing
    return bp
