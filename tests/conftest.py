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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The near-tie counts of every GPU parity comparison of the session (sequences that matched the oracle
    exactly, and those excused by a near tie the oracle recorded, per band)."""
    import parity_tally

    lines = parity_tally.summary_lines()
    if lines:
        terminalreporter.write_sep("-", "parity with the oracle (near ties counted, not failed)")
        for line in lines:
            terminalreporter.write_line(line)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()
