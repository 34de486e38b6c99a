import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden(name):
    """Rows of whitespace-separated fields from a golden file; '#' starts a comment."""
    rows = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
