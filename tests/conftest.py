import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _stale(lib, src):
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The CPU oracle is plain C; make sure its shared object matches its source."""
    from oracle import build as ob
    if _stale(ob.LIB, os.path.join(os.path.dirname(ob.LIB), "iqo.c")):
        ob.build()
    yield


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Rows of a whitespace-separated golden fixture, '#' lines skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows
