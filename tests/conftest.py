import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Every bf16 comparison of the session beside its rounding floor: the error of the
    HIP result and of the correctly rounded exact result, relative to each output
    vector's RMS, and the margin (2 delta) the element-wise bound allowed."""
    gu = sys.modules.get("tests.gpu_util")
    rows = getattr(gu, "BF16_REPORT", None) if gu else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "bf16 parity against the rounding floor (relative to each vector's RMS)")
    tr.write_line(f"{'comparison':80s} {'err max':>9s} {'floor max':>9s} {'err mean':>9s} "
                  f"{'floor mean':>10s} {'margin mean':>11s}")
    for what, mx, mean, fmx, fmean, mmx, mmean in rows:
        tr.write_line(f"{what[:80]:80s} {mx:9.3e} {fmx:9.3e} {mean:9.3e} {fmean:10.3e} {mmean:11.3e}")
    excess = max(r[2] - r[4] for r in rows)
    tr.write_line(f"{len(rows)} comparisons; largest mean excess over the floor {excess:.3e}")
