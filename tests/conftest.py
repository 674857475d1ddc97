"""Shared test set-up: the ``gpu`` marker, build-on-demand and fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU tests")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built here when no build exists yet or the source is newer)."""
    import oracle
    if not os.path.exists(oracle.LIB) or os.path.getmtime(oracle.LIB) < os.path.getmtime(oracle.SRC):
        oracle.build()
    return oracle.default()
