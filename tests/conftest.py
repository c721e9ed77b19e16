import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: 'name value rest...' lines, '#' comments."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if line.lstrip().startswith("#") else line.strip()
            if not line:
                continue
            parts = line.split()
            out[parts[0]] = parts[1:]
    return out


@pytest.fixture
def golden():
    return load_golden
