import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long exhaustive sweep, opt-in via MOE_EXHAUSTIVE=1")
    # the CPU oracle is test infrastructure: build its library variants when
    # they are missing or older than the source (loading it never compiles)
    import oracle
    stale = [v for v in oracle.VARIANTS if oracle.stale(v)]
    if stale:
        oracle.build(stale)


def pytest_collection_modifyitems(config, items):
    if os.environ.get("MOE_EXHAUSTIVE") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep; set MOE_EXHAUSTIVE=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)
