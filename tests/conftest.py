import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) device and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU-heavy oracle case (full-size shapes)")


@pytest.fixture(scope="session")
def cblib():
    """The fusor library; built in-tree first if it is missing."""
    from rag_kv_cache_layer_amd import fusor
    if not os.path.exists(fusor.LIB_PATH):
        from rag_kv_cache_layer_amd import build
        build.build()
    return fusor.lib()
