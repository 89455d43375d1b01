import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst output error of each named workload (and overall), printed even under -q."""
    try:
        import gpu_common
    except Exception:  # the CPU-only session never imports it
        return
    tr = terminalreporter
    frag = getattr(gpu_common, "FRAGILE", [])
    if frag:
        tr.write_sep("-", "mask parity: rows holding a fragile block")
        for group in ("config", "stage"):
            fs = [f for f in frag if f[0].startswith("config") == (group == "config")]
            if not fs:
                continue
            what, n, rows, bound = max(fs, key=lambda f: f[1] / max(f[2], 1))
            total = sum(f[1] for f in fs), sum(f[2] for f in fs)
            tr.write_line(f"{group + ' masks':13s} {len(fs)} mask heads, {total[0]} of {total[1]} rows "
                          f"({total[0] / max(total[1], 1):.2%}); worst head {n} of {rows} ({n / max(rows, 1):.1%}, "
                          f"bound {bound:.0%}) at {what}")
    errs = getattr(gpu_common, "ERRORS", [])
    if not errs:
        return
    tr.write_sep("-", "parity margins (worst error / bound)")
    groups = {}
    for what, metric, err, bound in errs:
        key = " ".join(what.split()[:2]) if what.startswith("config") else "stage tests"
        cur = groups.get((key, metric))
        if cur is None or err / bound > cur[1] / cur[2]:
            groups[(key, metric)] = (what, err, bound)
    for (key, metric), (what, err, bound) in sorted(groups.items()):
        tr.write_line(f"{key:12s} {metric:8s} worst {err:.3e} (bound {bound:.0e}, {err / bound:5.1%} of it) at {what}")
    tr.write_line(f"{len(errs)} output comparisons")
