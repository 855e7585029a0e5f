import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a `key = value` fixture from tests/golden into a dict of numbers."""
    values = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (p.strip() for p in line.split("=", 1))
            values[key] = float(val) if "." in val else int(val)
    return values


@pytest.fixture(scope="session")
def pages_capacity():
    return read_golden("pages_capacity.txt")
