import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: '#' comments, then whitespace-separated rows."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return read_golden


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Print the case name (flushed, uncaptured) before every GPU test runs."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.__stderr__.flush()
    yield
