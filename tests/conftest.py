import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def load_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    with open(path) as f:
        return [ln for ln in (l.split("#")[0].strip() for l in f) if ln]


@pytest.fixture(scope="session")
def golden():
    return load_golden
