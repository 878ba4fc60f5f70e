import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_runtest_logstart(nodeid, location):
    """GPU tests note each test's start in the progress file that the GPU
    helpers' log() writes (it stays quiet for CPU-only runs)."""
    if "test_gpu_" in nodeid or "test_zz_" in nodeid:
        from gpu_common import log
        log(f"[start] {nodeid}")
