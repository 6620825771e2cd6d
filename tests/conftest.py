import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The product binding on cuda:0.  Loud failure if the HIP library is
    missing or no GPU is visible: GPU tests never fall back to anything."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    import combine_moe_dispatch_layout_amd as moe
    moe.load_library()
    return moe
