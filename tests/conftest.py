import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running host work")


def pytest_terminal_summary(terminalreporter):
    """One line per output compared against the oracle or another entry point:
    raw max |error| (bars: bf16 1e-2 per element, fp32 1e-5), relative
    Frobenius error (bf16 bar 5e-3), and the worst error over the plain bar
    (bf16 max(1e-2, ulp), fp32 1e-5) and over the bar the test applied."""
    gc = sys.modules.get("gpu_common")
    recs = getattr(gc, "RECORDS", None) if gc else None
    if not recs:
        return
    tr = terminalreporter
    tr.section("compared outputs (raw error figures)")
    over = [r for r in recs if r[1] == "bf16" and r[2]["max_abs"] > 1e-2]
    over32 = [r for r in recs if r[1] == "fp32" and r[2]["max_abs"] > 1e-5]
    tr.write_line(f"{len(recs)} comparisons; {len(over)} bf16 ones with some element more than 1e-2 off "
                  "(allowed where one bf16 spacing of the exact value exceeds 1e-2); "
                  f"{len(over32)} fp32 ones with some element more than 1e-5 off (allowed only for K/V "
                  "heads that sum several attention gradients)")
    for name, dtype, st in recs:
        extra = ""
        if "max_err_over_unwidened" in st:
            flat = "1e-2" if dtype == "bf16" else "1e-5"
            extra = (f" over_plain {st['max_err_over_unwidened']:.3f} over_applied {st['max_err_over_allowed']:.3f}"
                     f" n_over_{flat} {st['n_over_flat']}")
        tr.write_line(f"  {name} [{dtype}, n={st['n']}]: max_abs {st['max_abs']:.3e} rel_fro {st['rel_fro']:.3e}"
                      + extra)
