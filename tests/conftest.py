import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


# Whole-output parity errors recorded by the GPU tests, printed in the
# terminal summary so that they show with `pytest -q` too.
PARITY_REPORT = []


def pytest_terminal_summary(terminalreporter):
    if PARITY_REPORT:
        terminalreporter.write_sep("-", "max-abs error against the fp64 oracle, whole outputs")
        for line in PARITY_REPORT:
            terminalreporter.write_line(line)
