import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_finish(session):
    """Start the oracle's worker processes, when a selected test uses them,
    before any test runs: workers are then never started from a process that
    has already initialised the GPU."""
    if any("oracle_pool_workers" in getattr(it, "fixturenames", ()) for it in session.items):
        import oracle_workers
        oracle_workers.start()


def pytest_unconfigure(config):
    mod = sys.modules.get("oracle_workers")
    if mod is not None:
        mod.stop()


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def oracle_pool_workers():
    """The oracle's host worker processes (tests/oracle_workers.py)."""
    import oracle_workers
    oracle_workers.start()
    return oracle_workers
