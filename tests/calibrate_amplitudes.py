"""Choose the field amplitudes of the video workloads (run by hand; not a test).

The block density that scoring + top-p produce depends on how peaked the strided-logit
softmax is, which scales with the Q/K field amplitude.  This script bisects the
amplitude until the oracle's mean density over a subset of heads lands on the target,
and prints the value that synthetic/workloads.py records (AMPLITUDE_CFG2, AMPLITUDE_CFG4).

    python tests/calibrate_amplitudes.py
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synthetic.workloads as sw  # noqa: E402
from oracle import pipeline  # noqa: E402


def mean_density(cfg: int, amplitude: float, heads) -> float:
    if cfg == 2:
        sw.AMPLITUDE_CFG2 = amplitude
    else:
        sw.AMPLITUDE_CFG4 = amplitude
    wl = sw.make_config(cfg, heads=heads, batches=[0])
    dens = []
    if wl.pool_gqa:
        for g in range(wl.Hkv):
            dens.append(pipeline.head_mask(wl, 0, g).mean())
    else:
        for h in range(wl.Hq):
            dens.append(pipeline.head_mask(wl, 0, h).mean())
    return float(np.mean(dens))


def bisect(cfg, target, lo, hi, heads, iters=7):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        d = mean_density(cfg, mid, heads)
        print(f"cfg{cfg} amplitude {mid:.4f} density {d:.4f}", flush=True)
        if d > target:
            lo = mid  # larger amplitude -> sharper softmax -> sparser
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    a2 = bisect(2, 0.22, 0.55, 0.9, heads=list(range(8)))
    a4 = bisect(4, 0.26, 0.85, 1.8, heads=list(range(10)))
    print(f"AMPLITUDE_CFG2 = {a2:.4f}\nAMPLITUDE_CFG4 = {a4:.4f}")
