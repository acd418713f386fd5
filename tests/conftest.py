import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library, through its Python binding (built first if absent)."""
    from learned_token_pruning_05_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from learned_token_pruning_05_amd import build as _build
        _build.build_library()
    return _lib.load()
