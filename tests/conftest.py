import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _built_checkers():
    """The oracle and the input generator are plain C built with gcc; build
    them once per session if their libraries are missing."""
    import oracle
    import synth
    if not os.path.exists(oracle._SO):
        oracle.build()
    if not os.path.exists(synth._SO):
        synth.build()
