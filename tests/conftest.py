import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle as o
    o.lib()
    return o


@pytest.fixture(scope="session")
def native():
    """The built HIP library on a visible GPU (built in-tree if absent)."""
    import torch
    from rank_markov_draft_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    if not os.path.exists(_lib.LIB_PATH):
        _lib.build()
    return _lib.load()
