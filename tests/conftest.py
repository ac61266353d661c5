import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # the CPU oracle is test infrastructure: build its library variants when
    # they are missing or older than the source (loading it never compiles)
    import oracle
    stale = [v for v in oracle.VARIANTS if oracle.stale(v)]
    if stale:
        oracle.build(stale)
