import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a golden text fixture: '#' comments, 'key ints...' lines, digit rows."""
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head = line.split()
            if head[0].isalpha():
                meta[head[0]] = [int(x) for x in head[1:]]
            else:
                rows.append([int(ch) for ch in line])
    return meta, rows
