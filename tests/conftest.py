import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst error against its bound for every GPU parity check that ran."""
    from tests import parity_log
    lines = parity_log.summary_lines()
    if not lines:
        return
    terminalreporter.section("parity: worst error per check")
    for ln in lines:
        terminalreporter.write_line(ln)
    parity_log.dump()
