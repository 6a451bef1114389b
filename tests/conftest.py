import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Parity margins recorded by the tests (name, measured, bound), printed in the
# terminal summary so that a quiet run (-q, no -s) still shows how close each
# full-size result came to its tolerance.
_MARGINS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture
def margin():
    def record(name, value, bound):
        _MARGINS.append((str(name), float(value), float(bound)))
        return value
    return record


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not _MARGINS:
        return
    terminalreporter.write_sep("-", "parity margins (measured / bound)")
    for name, v, b in _MARGINS:
        terminalreporter.write_line("%-58s %.3e / %.1e  (%3.0f%%)" % (name, v, b, 100.0 * v / b))
