import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_terminal_summary(terminalreporter):
    log = sys.modules.get("tests.gpu_common")
    log = getattr(log, "PARITY_LOG", None)
    if not log:
        return
    terminalreporter.section("parity: worst error vs bar")
    for test, what, err, bar in log:
        flag = "ok " if err <= bar else "OVER"
        terminalreporter.write_line(f"{flag} {err:9.3e} <= {bar:8.1e}  {test}: {what}")
