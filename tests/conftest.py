import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (large host memory and time)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Per-workload parity margins of the GPU layer tests (if any ran)."""
    mod = sys.modules.get("_gpu")
    rows = getattr(mod, "MARGINS", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "layer parity margins (max|gpu-oracle|/max|oracle|, every token)")
    for r in rows:
        tr.write_line("%-28s T=%-5d tokens %-5d tie flips %-3d rel err %.3g (tol %g)"
                      % (r["workload"], r["T"], r["compared"], r["tie_flips"], r["rel_err"],
                         r["tol"]))
