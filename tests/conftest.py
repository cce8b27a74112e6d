import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly if the device or the HIP library is missing; they
    # are only deselected by the marker expression, never silently skipped.
    pass


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle
