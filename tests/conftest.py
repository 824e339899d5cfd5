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
    "chunked" or "auto"): sets MSSM_SCAN_DESIGN, which the library reads at
    every call, and restores it afterwards."""
    old = os.environ.get("MSSM_SCAN_DESIGN")
    if request.param == "auto":
        os.environ.pop("MSSM_SCAN_DESIGN", None)
    else:
        os.environ["MSSM_SCAN_DESIGN"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("MSSM_SCAN_DESIGN", None)
    else:
        os.environ["MSSM_SCAN_DESIGN"] = old
