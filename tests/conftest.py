import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (host-only calls are safe without a GPU)."""
    from chunked_prefill_mixed_amd import build_lib, cpa
    if not __import__("os").path.exists(cpa.LIB_PATH):
        build_lib.build()
    return cpa.load()
