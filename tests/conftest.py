"""Shared fixtures.  Libraries are built once (``__graft_entry__.build()``) only if missing."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (runs through the C-ABI library on cuda:0)")
    config.addinivalue_line("markers", "slow: long CPU test")
    import __graft_entry__ as ge
    if not ge.all_built():
        ge.build()


@pytest.fixture(scope="session")
def root():
    return ROOT
