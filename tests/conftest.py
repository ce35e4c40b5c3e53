import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _parse_matrix(text, conv):
    rows = [r.split() for r in text.split("|")]
    return [[conv(v) for v in r] for r in rows]


def read_golden_sections(name):
    """Parse 'key = v v | v v' lines, grouped under optional [section] headers."""
    sections = {}
    cur = sections.setdefault("", {})
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = sections.setdefault(line[1:-1], {})
                continue
            key, _, val = line.partition("=")
            cur[key.strip()] = val.strip()
    return sections


@pytest.fixture
def golden():
    return read_golden_sections
