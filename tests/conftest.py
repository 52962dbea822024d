import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def pytest_collection_modifyitems(config, items):
    """GPU tests fail loudly when no GPU is visible: they are selected with
    -m gpu on a GPU machine and deselected with -m "not gpu" elsewhere."""
    return None


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle
