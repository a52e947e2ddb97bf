import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# Error figures of the parity tests (max|dO|, mean|dO|, max|dLSE| per case),
# printed in the terminal summary so that a run's log keeps them.
PARITY_FIGURES = []


@pytest.fixture
def parity_figures():
    return PARITY_FIGURES


def pytest_terminal_summary(terminalreporter):
    if not PARITY_FIGURES:
        return
    terminalreporter.section("parity error figures (against the fp64 oracle)")
    for line in PARITY_FIGURES:
        terminalreporter.write_line(line)
