import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_WORKLOADS = {}


@pytest.fixture(scope="session")
def workload_cache():
    """Session cache of generated workloads: generation of the large-model
    weights takes seconds, so tests share them by key."""
    return _WORKLOADS
