import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than ~10 s")


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import ref
    return ref.lib()


def pytest_sessionfinish(session, exitstatus):
    """Write the worst attention errors seen by the GPU parity tests (if any ran)."""
    try:
        from kivi_testlib import REPORT
    except Exception:
        return
    if REPORT:
        import json
        out = os.path.join(ROOT, "gpurun_out")
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "parity_report.json"), "w") as f:
            json.dump(dict(sorted(REPORT.items())), f, indent=1)
