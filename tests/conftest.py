import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size parity cases (minutes of oracle time)")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


@pytest.fixture(autouse=True)
def _parity_case_name(request):
    """Names the recorded parity ratios after the running test."""
    mod = sys.modules.get("gpu_parity_helpers")
    if mod is not None:
        mod.set_case(request.node.name)
    yield


def pytest_sessionfinish(session, exitstatus):
    """With $MOE_PARITY_REPORT set, write max |gpu - oracle| / (atol + rtol
    |oracle|) at the stated tolerance for every output the GPU tests
    compared (JSON, keyed test:output)."""
    path = os.environ.get("MOE_PARITY_REPORT")
    mod = sys.modules.get("gpu_parity_helpers")
    if path and mod is not None and mod.RATIOS:
        import json
        with open(path, "w") as f:
            json.dump(mod.RATIOS, f, indent=1, sort_keys=True)
