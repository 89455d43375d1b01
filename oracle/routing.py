"""Error-aware block routing (oracle; test infrastructure only).

Pages:
  [SBC] "Sparse-block compensation", section "SVG-EAR -- centroid compensation": skipped
        keys are replaced by their cluster centroid inside one softmax, and the method adds a
        router that picks the blocks to compute exactly; section "Out of scope, and why"
        calls that router a policy on top of the compensated primitive.
  [BSA] "Block-sparse attention" topic page, the SVG-EAR card (abstract): centroid
        compensation is accurate for most blocks but fails on a few; selecting blocks by
        attention score says where the mass is, not where the approximation error is; a
        lightweight probe estimates each block's compensation error, and the blocks with the
        highest error-to-cost ratio are computed exactly while the rest are compensated.

The pages give no formula for the probe, the error or the budget.  Readings (the plainest
ones the rest of the pages support):
  * Probe.  One probe per query cluster a: its centroid q_bar_a, the mean of the cluster's
    query rows (the query-side counterpart of k_bar_c), here in float64.  Empty query clusters
    get a zero probe and no route.  (A kernel may hand its probes to the error pass in the
    input type; parity then compares within that rounding.)
  * Error.  For the probe, with logits s_j = q_bar_a . k_j * scale over all keys, softmax
    weights p_j = exp(s_j - lse) and dense output O_a = sum_j p_j v_j: compensating block
    (a, c) alone replaces the cluster's exact terms (N_c = sum_{j in c} p_j v_j,
    Z_c = sum_{j in c} p_j) by the centroid column (z_hat = exp(q_bar_a . k_bar_c * scale
    + log n_c - lse), N_hat = z_hat v_bar_c).  To first order the probe's output then moves
    by  delta = (N_hat - N_c) - O_a (z_hat - Z_c);  the block's compensation error is the
    Euclidean norm of delta.  (The exact change is delta / (1 + z_hat - Z_c); the first-order
    form is what adds over blocks.)  Empty key clusters have no error and no cost.
  * Cost.  Computing block (a, c) exactly costs n_a * n_c token pairs; within a row a the
    ratio error / cost orders the clusters as error / n_c.
  * Budget.  Each row keeps the shortest prefix of its non-empty clusters, ordered by
    error / n_c descending (ties: lower cluster index first), whose key count reaches
    `budget` tokens (the caller's density times the key count), and at least one cluster;
    every other cluster is compensated by the attention.
"""

from __future__ import annotations

import numpy as np


def query_centroids(q, q_labels, Cq: int) -> np.ndarray:
    """Probe rows q_bar [B, Hq, Cq, D] in float64: the mean of each query cluster's rows
    (zero for an empty cluster)."""
    q = np.asarray(q, dtype=np.float64)
    lab = np.asarray(q_labels)
    B, H, S, D = q.shape
    out = np.zeros((B, H, Cq, D))
    for a in range(Cq):
        rows = np.nonzero(lab == a)[0]
        if rows.size:
            out[:, :, a, :] = q[:, :, rows, :].mean(axis=2)
    return out


def block_compensation_error(qbar, k, v, k_labels, Ck: int, scale: float) -> np.ndarray:
    """err [B, Hq, Cq, Ck]: the first-order output error of compensating each block for the
    probe q_bar_a (see the header).  K/V heads are shared by Hq // Hkv query heads."""
    qbar = np.asarray(qbar, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lab = np.asarray(k_labels)
    B, Hq, Cq, D = qbar.shape
    G = Hq // k.shape[1]
    members = [np.nonzero(lab == c)[0] for c in range(Ck)]
    err = np.zeros((B, Hq, Cq, Ck))
    for b in range(B):
        for h in range(Hq):
            K, V = k[b, h // G], v[b, h // G]
            kbar = np.array([K[m].mean(axis=0) if m.size else np.zeros(D) for m in members])
            vbar = np.array([V[m].mean(axis=0) if m.size else np.zeros(D) for m in members])
            for a in range(Cq):
                s = K @ qbar[b, h, a] * scale
                mx = s.max()
                lse = mx + np.log(np.exp(s - mx).sum())
                p = np.exp(s - lse)
                O = p @ V
                for c, m in enumerate(members):
                    if m.size == 0:
                        continue
                    Zc = p[m].sum()
                    Nc = p[m] @ V[m]
                    zhat = np.exp(qbar[b, h, a] @ kbar[c] * scale + np.log(m.size) - lse)
                    delta = (zhat * vbar[c] - Nc) - O * (zhat - Zc)
                    err[b, h, a, c] = np.sqrt(delta @ delta)
    return err


def error_aware_route(err, k_counts, budget: float) -> np.ndarray:
    """Keep bits uint8 [B, H, Cq, Ck]: per row, the shortest prefix of the non-empty clusters
    in order of err / n_c (descending, ties by index) whose key count reaches `budget`, and
    at least one cluster (see the header).  Ratios are formed in float64."""
    err = np.asarray(err, dtype=np.float64)
    n = np.asarray(k_counts, dtype=np.int64)
    keep = np.zeros(err.shape, dtype=np.uint8)
    nz = np.nonzero(n > 0)[0]
    for idx in np.ndindex(*err.shape[:-1]):
        row = err[idx]
        ratio = row[nz] / n[nz].astype(np.float64)
        order = nz[np.lexsort((nz, -ratio))]  # descending ratio, lower index first on ties
        total = 0
        for c in order:
            keep[idx + (c,)] = 1
            total += n[c]
            if total >= budget:
                break
    return keep
