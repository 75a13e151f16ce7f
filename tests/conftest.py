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
    config.addinivalue_line("markers", "slow: large host-side oracle work (minutes)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    from helpers import PARITY
    if not PARITY:
        return
    terminalreporter.write_sep("-", "rel-L2 against the oracle (case: value / bound)")
    for case, err, bound in PARITY:
        terminalreporter.write_line(f"{case}: {err:.3e} / {bound:g}")
