import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU time")


def pytest_terminal_summary(terminalreporter):
    """The achieved error of every attention comparison of the run."""
    mod = sys.modules.get("gpu_util")
    margins = getattr(mod, "MARGINS", None) if mod else None
    if not margins:
        return
    tr = terminalreporter
    tr.section("attention parity margins (|gpu - oracle|; pass: err <= 2e-3 + 1e-2 |oracle|)")
    tr.write_line(f"{'max-abs':>10} {'max-rel':>10} {'err/bound':>9} {'elements':>10}  case")
    for r in margins:
        tr.write_line(f"{r['max_abs']:10.3e} {r['max_rel_ref_ge_0.2']:10.3e} {r['max_err_over_bound']:9.4f} "
                      f"{r['elements']:10d}  {r['case']}")
    worst = max(margins, key=lambda r: r["max_abs"])
    tr.write_line(f"largest max-abs {worst['max_abs']:.3e} ({worst['case']}); "
                  f"{sum(r['elements'] for r in margins)} elements in {len(margins)} comparisons")
