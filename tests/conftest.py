import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libkda.so")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def ref():
    """The fp64 oracle (built on first use)."""
    import oracle
    return oracle.kda_reference


def pytest_terminal_summary(terminalreporter):
    """The parity line of every GPU comparison (whole-tensor, worst head, worst row), so
    that they appear in the log of a quiet run too."""
    try:
        from kda_testlib import PARITY_LOG
    except ImportError:
        return
    if PARITY_LOG:
        terminalreporter.section("parity: whole tensor, worst (sequence, head), worst row")
        for line in PARITY_LOG:
            terminalreporter.write_line(line)
