import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def workloads():
    """Session cache of drawn workloads (the large weights take seconds to draw)."""
    from mtp_draft_head_amd import inputs

    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = inputs.make(name)
        return cache[name]

    return get
