import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def page_figures():
    import json
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return json.load(f)


def pytest_terminal_summary(terminalreporter):
    import parity_log
    lines = parity_log.summary_lines()
    if lines:
        terminalreporter.section("parity: measured max-abs errors")
        for line in lines:
            terminalreporter.write_line(line)
