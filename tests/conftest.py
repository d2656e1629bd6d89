import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host time)")


@pytest.fixture(scope="session")
def hip():
    """The HIP library binding on cuda:0; GPU tests fail loudly if it cannot load."""
    import torch

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import grouped_nvfp4_w4a16_amd as m

    m.load()  # raises if the shared library is missing
    return m
