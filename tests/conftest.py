import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)


def pytest_sessionstart(session):
    """Build liblh.so in-tree when nothing is built yet (a built library is used as is)."""
    from hierarchical_sparse_attention_lh_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from hierarchical_sparse_attention_lh_amd import build
        build.build()
