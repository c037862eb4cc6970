import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle

    return oracle.load()


@pytest.fixture(scope="session")
def native():
    """The C-ABI library, built in-tree with hipcc first if it is missing or
    older than its sources (the digest the build recorded beside it)."""
    from tiled_dense_gemm_scale_amd import _native, build

    if build.is_stale(_native.LIBRARY):
        build.build(_native.LIBRARY)
    return _native
