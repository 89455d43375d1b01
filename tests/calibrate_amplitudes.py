"""Choose the field amplitudes of the video workloads (run by hand; not a test).

The block density that scoring + top-p produce depends on how peaked the strided-logit
softmax is, which scales with the Q/K field amplitude.  This script bisects the amplitude
until the oracle's kept-pair density over every mask head of the workload (every batch
entry) lands on the target, and prints the value that synthetic/workloads.py records
(AMPLITUDE_CFG2, AMPLITUDE_CFG4).  Kept-pair density is the number of token pairs in kept
blocks over S^2, averaged over mask heads.

    python tests/calibrate_amplitudes.py [2|4]
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synthetic.workloads as sw  # noqa: E402
from oracle import pipeline  # noqa: E402
from oracle.layout import cluster_layout  # noqa: E402


def pair_density(wl) -> float:
    _, _, counts = cluster_layout(wl.labels, wl.C)
    n = counts.astype(np.float64)
    dens = []
    for b in range(wl.B):
        for hm in range(wl.Hm):
            keep = pipeline.head_mask(wl, b, hm).astype(np.float64)
            dens.append(float(n @ keep @ n) / float(wl.S) ** 2)
    return float(np.mean(dens))


def density_at(cfg: int, amplitude: float) -> float:
    if cfg == 2:
        sw.AMPLITUDE_CFG2 = amplitude
    else:
        sw.AMPLITUDE_CFG4 = amplitude
    return pair_density(sw.make_config(cfg))


def bisect(cfg, target, lo, hi, iters=8):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        d = density_at(cfg, mid)
        print(f"cfg{cfg} amplitude {mid:.4f} kept-pair density {d:.4f}", flush=True)
        if d > target:
            lo = mid  # larger amplitude -> sharper softmax -> sparser
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    which = [int(a) for a in sys.argv[1:]] or [2, 4]
    if 2 in which:
        print(f"AMPLITUDE_CFG2 = {bisect(2, 0.22, 0.5, 0.8):.4f}", flush=True)
    if 4 in which:
        print(f"AMPLITUDE_CFG4 = {bisect(4, 0.26, 0.7, 1.1):.4f}", flush=True)
