import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    """The CPU oracle, built from source if the library is missing."""
    import oracle
    from oracle import build as oracle_build
    if not os.path.exists(oracle.LIB_PATH):
        oracle_build.build()
    oracle.load()
    return oracle
