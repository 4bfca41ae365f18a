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
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """The GEMM error measure over every product comparison of the session: the floored
    relative error (the pass bar), the plain normwise error and the floor-clamped count."""
    try:
        from helpers import P2_RECORDS
    except ImportError:
        return
    if not P2_RECORDS:
        return
    tr = terminalreporter
    worst = max(P2_RECORDS, key=lambda r: r[1])
    worst_n = max(P2_RECORDS, key=lambda r: r[2])
    clamped = sum(r[3] for r in P2_RECORDS)
    total = sum(r[4] for r in P2_RECORDS)
    tr.write_sep("-", "GEMM error (floored relative / normwise) over product comparisons")
    tr.write_line(f"comparisons: {len(P2_RECORDS)}, outputs compared: {total}, below the 1e-3 max|y*| floor: {clamped}")
    tr.write_line(f"worst floored relative error: {worst[1]:.3e} ({worst[0]})")
    tr.write_line(f"worst normwise max|dy|/max|y*|: {worst_n[2]:.3e} ({worst_n[0]})")
