import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


@pytest.fixture(scope="session")
def pivot_lib():
    """libpivot.so, built in-tree first if nothing is built yet."""
    import sparse_attention_indexer_proxy_amd as pv
    if not os.path.exists(pv.library_path()):
        from sparse_attention_indexer_proxy_amd import build
        build.build()
    return pv.load_library()
