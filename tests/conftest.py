import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-side oracle runs")


def pytest_runtest_logreport(report):
    """Print a failure's traceback as soon as it happens, so the cause stays in
    the log even if a later test ends the process."""
    if report.failed and report.when == "call":
        print(f"\n---- FAILED {report.nodeid}\n{report.longreprtext[-3000:]}\n----", flush=True)
