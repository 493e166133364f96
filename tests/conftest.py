import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-oracle cases")


def pytest_terminal_summary(terminalreporter):
    # decision flips between the GPU and the oracle seen by the parity checks, per input dtype
    parity = sys.modules.get("tests.parity")
    tally = getattr(parity, "FLIP_TALLY", None)
    if tally:
        terminalreporter.write_line("decision flips vs the oracle (pairs compared, |margin| <= 1e-3, wider): " + "; ".join(
            f"{dt}: {int(t['pairs'])}, {int(t['tight'])}, {int(t['wide'])}" for dt, t in sorted(tally.items())))
