import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def load_golden():
    return golden


def ensure_library():
    """Build libcsa.so if it is missing or was built from other sources than
    the tree's (its embedded source digest differs); hipcc cross-compiles on
    the CPU, so a stale library is never the one under test."""
    import __graft_entry__
    return __graft_entry__._build_module().ensure_current()
