"""Cluster centroids and counts (oracle).

[SBC] "SVG-EAR -- centroid compensation": every skipped key is replaced by the centroid of
its cluster and its value by the cluster's value centroid; a cluster's keys then share one
logit and collapse to one term weighted by the cluster size n_c.
"""

from __future__ import annotations

import numpy as np


def centroids(k: np.ndarray, v: np.ndarray, labels: np.ndarray, C: int):
    """Per-cluster means of keys and values, and cluster sizes.

    k, v: [S, D]; labels: [S] in [0, C).  Returns (kbar [C, D], vbar [C, D], n [C]) in
    float64.  An empty cluster has n = 0 and zero centroids (its compensation term then
    carries log 0 = -inf and vanishes).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    D = k.shape[1]
    n = np.zeros(C, dtype=np.int64)
    ksum = np.zeros((C, D))
    vsum = np.zeros((C, v.shape[1]))
    for c in range(C):
        members = labels == c
        n[c] = int(members.sum())
        ksum[c] = k[members].sum(axis=0)
        vsum[c] = v[members].sum(axis=0)
    safe = np.maximum(n, 1)[:, None]
    kbar = np.where(n[:, None] > 0, ksum / safe, 0.0)
    vbar = np.where(n[:, None] > 0, vsum / safe, 0.0)
    return kbar, vbar, n
