import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    """Parse a `key: v1 v2 ...` fixture file; `#` starts a comment; keys may repeat."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split(":", 1)
            toks = []
            for t in vals.split():
                toks.append(int(t, 16) if t.lower().startswith(("0x", "-0x")) else
                            (int(t) if t.lstrip("-").isdigit() else float(t)))
            out.setdefault(key.strip(), []).append(toks)
    return out


@pytest.fixture
def golden():
    return load_golden
