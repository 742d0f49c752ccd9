import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def pytest_sessionfinish(session, exitstatus):
    """Writes the largest error of every recorded parity case (GPU runs) to
    gpurun_out/parity_max_err.json, so the margins survive a quiet run."""
    mod = sys.modules.get("tests.paged_case")
    errors = getattr(mod, "ERRORS", None)
    if not errors:
        return
    out_dir = os.path.join(ROOT, "gpurun_out")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "parity_max_err.json"), "w") as f:
        json.dump(dict(sorted(errors.items())), f, indent=1)
