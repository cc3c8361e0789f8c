import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session", autouse=True)
def _native_test_libs():
    """The oracle and the input generator are plain C built with gcc; build
    them if a checkout has not yet done so."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(synth.LIB_PATH):
        synth.build()
    yield
