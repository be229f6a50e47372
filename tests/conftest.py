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
    """Rows of a whitespace-separated golden table; '#' starts a comment line."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split(None, 2))
    return rows


def parse_num(tok):
    t = tok.strip()
    neg = t.startswith("-")
    body = t[1:] if neg else t
    v = float.fromhex(body) if body.lower().startswith("0x") else float(body)
    return -v if neg else v


@pytest.fixture(scope="session")
def golden():
    return read_golden
