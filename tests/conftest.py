import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def read_golden(name):
    """Parse a tests/golden text fixture into {section: list of rows}."""
    return read_golden_path(os.path.join(ROOT, "tests", "golden", name))


def read_golden_path(path):
    sections, cur = {}, None
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if len(parts) == 1 and not _isnum(parts[0]):
                cur = parts[0]
                sections[cur] = []
            else:
                sections.setdefault(cur, []).append(parts)
    return sections


def _isnum(s):
    try:
        float(s)
        return True
    except ValueError:
        return False


@pytest.fixture(scope="session")
def golden():
    return read_golden
