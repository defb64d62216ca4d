import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; the GPU tests themselves are marked `gpu`."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per comparison of GPU output against the oracle: how far the worst element went past the
    stated per-element bound, as a fraction of the floor in force and of 2**-20 absum. Written to
    the file named by BFP8_TOL_REPORT as JSON when that is set."""
    from tests import tolerance

    if not tolerance.RECORDS:
        return
    path = os.environ.get("BFP8_TOL_REPORT")
    if path:
        tolerance.write_report(path)
    tr = terminalreporter
    tr.section("GEMM tolerance: worst excess over the stated bound, per comparison")
    worst_floor = max(r["worst_over_floor"] for r in tolerance.RECORDS)
    worst_absum = max(r["worst_over_absum"] for r in tolerance.RECORDS)
    over = sum(r["over_stated"] for r in tolerance.RECORDS)
    total = sum(r["n"] for r in tolerance.RECORDS)
    tr.write_line(f"{len(tolerance.RECORDS)} comparisons, {total} elements, {over} over the stated bound; "
                  f"worst excess / floor in force = {worst_floor:.4g}, worst excess / (2^-20 absum) = {worst_absum:.4g}")
    for r in sorted(tolerance.RECORDS, key=lambda r: -r["worst_over_absum"])[:40]:
        tr.write_line(f"  {r['worst_over_absum']:9.4g} {r['worst_over_floor']:9.4g} {r['over_stated']:6d}/{r['n']:<8d} "
                      f"{r['what']}  [{r['test']}]")
