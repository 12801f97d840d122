import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C ABI")


def pytest_make_parametrize_id(config, val, argname):
    # shapes read in test ids: (1, 1, 300, 256) -> 1x1x300x256
    if isinstance(val, tuple) and val and all(isinstance(x, int) for x in val):
        return "x".join(str(x) for x in val)
    return None


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Lines of a golden fixture without comments, split into fields."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                rows.append(ln.split())
    return rows


@pytest.fixture
def golden():
    return read_golden
