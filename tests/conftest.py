import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_golden(name):
    """Parse a golden text fixture: '# comments', '[section]' headers and
    'key: values' lines; matrices use '|' between rows."""
    sections = {}
    cur = sections.setdefault("", {})
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = sections.setdefault(line[1:-1], {})
                continue
            key, val = line.split(":", 1)
            rows = [r.split() for r in val.split("|")]
            arr = np.array([[float(v) for v in r] for r in rows])
            cur[key.strip()] = arr if len(rows) > 1 else arr[0]
    return sections


@pytest.fixture
def golden():
    return read_golden
