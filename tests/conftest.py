import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU work (oracle at full size)")


@pytest.fixture(autouse=True)
def _parity_test_id(request):
    """Names the running test in the parity margins (tests/parity_util.py)."""
    pu = sys.modules.get("tests.parity_util")
    if pu is not None:
        pu.CURRENT_TEST[0] = request.node.name
    yield


def pytest_sessionfinish(session, exitstatus):
    """Parity margins of the GPU tests that ran, written under gpurun_out/."""
    pu = sys.modules.get("tests.parity_util")
    if pu is not None and pu.MARGINS:
        pu.write_margins(os.path.join(ROOT, "gpurun_out", "parity_margins.md"))
