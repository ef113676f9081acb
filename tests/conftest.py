import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run in a fixed, cheap-first order inside one process.
    pass


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
