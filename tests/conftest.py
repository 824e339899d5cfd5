import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "page_examples.json")) as f:
        return json.load(f)


@pytest.fixture
def design(request):
    """Pins the scan order for one test (parametrize indirectly with "chain",
    "chunked" or "auto") through the library's tuning setting, restored
    afterwards."""
    from selective_state_space_54_amd import mssm
    with mssm.tuning(scan_order=request.param):
        yield request.param


@pytest.fixture
def chunk_len(request):
    """Forces the chunked order's chunk length (None: automatic) for one test,
    through the library's tuning setting; exercises the chunk carries."""
    from selective_state_space_54_amd import mssm
    with mssm.tuning(chunk_len=request.param or 0):
        yield request.param
