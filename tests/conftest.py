import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of host work")


def pytest_terminal_summary(terminalreporter):
    """Observed errors of the GPU parity checks against their bounds (every workload)."""
    gh = sys.modules.get("tests.gpu_helpers")
    errs = getattr(gh, "ERRS", None) if gh else None
    if not errs:
        return
    tr = terminalreporter
    tr.write_sep("-", f"float parity: max row relative error of {len(errs)} checks")
    worst = {}
    for label, err, tol in errs:
        if label not in worst or err / tol > worst[label][0] / worst[label][1]:
            worst[label] = (err, tol)
    for label, (err, tol) in sorted(worst.items()):
        tr.write_line(f"{label:58s} {err:9.3e}  bound {tol:7.1e}  ({100 * err / tol:5.1f}%)")
