import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the oracle and the synthetic-input library only when they are missing."""
    import oracle.build
    import synth.build
    if not os.path.exists(oracle.build.LIB):
        oracle.build.build()
    if not os.path.exists(synth.build.LIB):
        synth.build.build()


_ensure_built()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle
