import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle runs that take tens of seconds on the host")


def read_golden(name: str) -> dict:
    """key = value lines (comma-separated floats allowed); '#' starts a comment."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [float(x) for x in val.split(",")]
            out[key] = vals if len(vals) > 1 else vals[0]
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden
