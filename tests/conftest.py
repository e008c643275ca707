import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.hookimpl(trylast=True)
def pytest_collection_modifyitems(session, config, items):
    """Fork the reference pool when a selected test uses it, before any test runs (and so before
    any test initialises the GPU runtime: a process that has must not fork)."""
    if any("oracle_pool" in getattr(it, "fixturenames", ()) for it in items):
        from tests import oracle_pool
        oracle_pool.start()


def pytest_unconfigure(config):
    mod = sys.modules.get("tests.oracle_pool")
    if mod is not None:
        mod.stop()


@pytest.fixture(scope="session")
def oracle_pool():
    from tests import oracle_pool as op
    return op.pool()
