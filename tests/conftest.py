import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """Skips only where no GPU is visible; on a GPU machine the HIP library must
    load (the package raises if it is missing)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import combine_ep_get_layout_amd as ep
    ep.load_library()
    return ep
