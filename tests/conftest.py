import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP library loaded on cuda:0)")
    config.addinivalue_line("markers", "slow: long CPU-side check")


@pytest.fixture(autouse=True)
def _gpu_test_progress(request):
    """Note each GPU test's start and end in gpurun_out/gpu_test_progress.log
    (pytest holds a test's own output back until it ends)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import time
    path = os.path.join(ROOT, "gpurun_out", "gpu_test_progress.log")

    def note(what):
        try:
            os.makedirs(os.path.dirname(path), exist_ok=True)
            with open(path, "a") as f:
                f.write(f"{time.strftime('%H:%M:%S')} {what} {request.node.nodeid}\n")
        except OSError:
            pass
    note("start")
    yield
    note("end")
