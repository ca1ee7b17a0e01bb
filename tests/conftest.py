import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """The parity cases' statistics (indices that differ from the oracle's,
    near ties, blocks passing only through the fp32 allowance, worst
    deviations), also when pytest captured the tests' output."""
    import parity
    if parity.SUMMARY:
        terminalreporter.section("parity against the oracle")
        for line in parity.SUMMARY:
            terminalreporter.write_line(line)
