import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

import _report  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a gfx950 GPU and the built HIP library (run on an MI355X)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if _report.LINES:
        terminalreporter.section("parity statistics (worst error/tolerance ratios, near-tie branches, slack)")
        for line in _report.LINES:
            terminalreporter.write_line(line)
