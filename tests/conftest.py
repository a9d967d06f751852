import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# Figures the parity tests record (flagged and mismatched windows, error ratios), printed
# at the end of the session so that they appear in the log of a quiet run too.
REPORT = []


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if REPORT:
        terminalreporter.write_sep("-", "parity figures")
        for line in REPORT:
            terminalreporter.write_line(line)
