import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_report_header(config):
    """Names the library the run loads and the sources it was built from: load() refuses a
    library whose compiled-in source hash differs from the sources on disk."""
    from grouped_nvfp4_w4a16_amd import LIB_PATH, build

    on_disk = build.source_sha256()
    if not os.path.exists(LIB_PATH):
        return f"libmoe_w4a16.so: not built (sources {on_disk[:16]})"
    import ctypes

    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_w4a16_source_sha256.restype = ctypes.c_char_p
    built = lib.moe_w4a16_source_sha256().decode()
    state = "matches the sources on disk" if built == on_disk else "STALE: differs from the sources"
    return f"libmoe_w4a16.so: built from sources {built[:16]} ({state})"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host time)")


@pytest.fixture(scope="session")
def hip():
    """The HIP library binding on cuda:0; GPU tests fail loudly if it cannot load."""
    import torch

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import grouped_nvfp4_w4a16_amd as m

    m.load()  # raises if the library is missing or was built from other sources
    return m
