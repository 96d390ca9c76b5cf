import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def pytest_sessionfinish(session, exitstatus):
    """Write the parity margins the GPU tests recorded (nothing on CPU runs)."""
    try:
        import parity_log
    except ImportError:
        return
    parity_log.dump(os.path.join(ROOT, "gpurun_out", "parity_margins.json"))
