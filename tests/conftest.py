import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Non-comment lines of a golden fixture, split at ':' into (head tokens, values)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                head, vals = line.split(":", 1)
                rows.append(([int(x) for x in head.split()], [int(x) for x in vals.split()]))
            else:
                rows.append((line.split(), None))
    return rows


@pytest.fixture
def golden():
    return read_golden
