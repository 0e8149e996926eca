import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a golden fixture: '#' comments, 'key = value' lines; values are floats or
    whitespace-separated float lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(x) for x in v.split()]
            out[k] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture
def golden():
    return read_golden
