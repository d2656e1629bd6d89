import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_report_header(config):
    """Names the sources the library was built from (read from the file, not loaded: torch
    must load its HIP runtime first). load() refuses a library whose compiled-in source
    hash differs from the sources on disk."""
    from grouped_nvfp4_w4a16_amd import build

    on_disk = build.source_sha256()
    built = build.built_source_sha256()
    if built is None:
        return f"libmoe_w4a16.so: not built (sources {on_disk[:16]})"
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
