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


@pytest.fixture(autouse=True)
def guard_bands(request):
    """GPU tests: every buffer the binding allocates gets canary guard bands (kivi_testlib.Guard),
    checked after every library call and at the end of the test."""
    if request.node.get_closest_marker("gpu") is None:
        yield None
        return
    import torch
    if not torch.cuda.is_available():
        yield None
        return
    from kivi_testlib import Guard
    from kv_cache_bit_quantize_amd import kivi
    guard = Guard()
    check = kivi._check

    def checked(status, where):
        check(status, where)
        guard.check(where)

    mp = pytest.MonkeyPatch()
    mp.setattr(kivi, "_zeros", guard.zeros)
    mp.setattr(kivi, "_empty", guard.empty)
    mp.setattr(kivi, "_check", checked)
    try:
        yield guard
    finally:
        mp.undo()
    guard.check("the test")


def pytest_sessionfinish(session, exitstatus):
    """Write the worst attention errors seen by the GPU parity tests (if any ran) to the json
    file KIVI_PARITY_REPORT names (nothing when it is unset)."""
    try:
        from kivi_testlib import REPORT
    except Exception:
        return
    path = os.environ.get("KIVI_PARITY_REPORT")
    if REPORT and path:
        import json
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(dict(sorted(REPORT.items())), f, indent=1)
