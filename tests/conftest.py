import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    # a fresh checkout has no built library (it is not versioned): build it once
    # here (hipcc cross-compiles without a GPU) rather than in whichever test
    # happens to need it first
    import soft_voronoi_render_amd as sad
    if not os.path.exists(sad.LIB_PATH):
        sad.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    oracle.set_threads(min(8, os.cpu_count() or 1))
    return oracle
