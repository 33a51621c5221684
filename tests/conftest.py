import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) device and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def read_golden(name):
    """Parse a tests/golden fixture into {key: [values...]} (repeated keys append)."""
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out.setdefault(key.strip(), []).append(val.strip())
    return out


def hexbytes(s):
    import numpy as np
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
