import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _native_helpers():
    """Make sure the CPU-side helper libraries (generators, oracle) exist."""
    import oracle
    import synth

    if not os.path.exists(synth._LIB_PATH):
        synth.build()
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    yield
