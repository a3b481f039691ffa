import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def read_golden(name):
    """Rows of a whitespace-separated fixture under tests/golden/, comments dropped."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return read_golden
