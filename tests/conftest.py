import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import parity_margins  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity error margins of the session (GPU tests only record any)."""
    lines = parity_margins.lines(2e-2, 5e-3)
    if lines:
        terminalreporter.write_sep("-", "parity margins (bar / error)")
        for ln in lines:
            terminalreporter.write_line(ln)
