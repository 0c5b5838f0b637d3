import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size shapes (minutes on CPU)")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def read_golden(name):
    """Key/value lines of a golden fixture, comments (#) dropped; repeated keys accumulate."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line and not line.startswith("0x"):
                k, v = line.split(":", 1)
                out.setdefault(k.strip(), []).append(v.strip())
            else:
                out.setdefault("_rows", []).append(line)
    return out
