import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


@pytest.fixture
def rng(request):
    """A generator seeded from the test's own id, so a test's inputs do not depend on which other
    tests ran before it."""
    import zlib

    import numpy as np
    return np.random.default_rng(zlib.crc32(request.node.nodeid.encode()))
