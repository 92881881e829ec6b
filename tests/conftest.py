import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: '# ...' comments, 'key: v v v' lines."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            toks = val.split()
            conv = []
            for t in toks:
                try:
                    conv.append(int(t))
                except ValueError:
                    conv.append(t)
            out[key.strip()] = conv
    return out


@pytest.fixture
def golden():
    return load_golden
