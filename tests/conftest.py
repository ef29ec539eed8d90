import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libcpattn.so")


def read_golden(name):
    """Rows of a golden fixture: lists of ints after the 'key:' prefix (or whole
    lines of ints), comments and blank lines skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                key, vals = line.split(":", 1)
                rows.append((int(key), [int(v) for v in vals.split()]))
            else:
                rows.append([int(v) for v in line.split()])
    return rows


@pytest.fixture
def golden():
    return read_golden
