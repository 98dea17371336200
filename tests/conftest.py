import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    mod = sys.modules.get("sa_testutil")
    log = getattr(mod, "PARITY_LOG", None) if mod is not None else None
    if log:
        terminalreporter.write_sep("-", "achieved parity errors (max|gpu - ref| / max|ref|)")
        for line in log:
            terminalreporter.write_line(line)
