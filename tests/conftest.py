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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_terminal_summary(terminalreporter):
    import parity_log
    if parity_log.RECORDS:
        terminalreporter.write_sep("-", "parity exemptions (excused / compared)")
        for line in parity_log.lines():
            terminalreporter.write_line(line)
