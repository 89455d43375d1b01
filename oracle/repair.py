"""SparsePR probe-fitted residual repair (oracle).

[SPR] (Probe-Fitted Residual Reconstruction paragraph): M query rows (64 by default) get
exact dense attention; the residual R = O_dense - O_sparse on those rows is fitted by a
weighted ridge regression (lambda = 0.1) from the standardized sparse output; the
feature-dependent part of the correction is projected on the top r = 16 principal
directions of the probe residuals; the correction is then applied to every row.  The
fit runs on every call, per (batch, head).  [SBC] "SparsePR -- probe-fitted residual
repair" says the same; [SBC] "Deviations from the papers": probes are the middle-out
member of each query cluster, chosen round-robin over clusters with weights |G_a| / m_a,
and the weights are normalized to sum to 1.

Readings taken where the pages are silent (each is the plainest one the text supports):
  * standardization uses the weighted mean and standard deviation of the probe rows
    (a deviation below 1e-6 counts as 1);
  * the intercept is the weighted mean residual: fitted without penalty and not
    projected (only the feature-dependent correction is projected);
  * "principal residual directions" are the leading eigenvectors of the weighted
    covariance of the centered probe residuals; directions with no energy (eigenvalue
    at most 1e-12 of the largest) are dropped, so fewer than r may be used;
  * the correction is added to every row, probe rows included (they are not overwritten);
  * when M is smaller than the number of query clusters, the single round of probes is
    spread evenly over the clusters (cluster floor((k + 1/2) * C / M) for k < M) instead of
    taking the first M clusters; later rounds visit clusters in index order.
"""

from __future__ import annotations

import numpy as np
import scipy.linalg


def middle_out(n: int):
    """Member order inside a cluster of n rows: m, m-1, m+1, m-2, m+2, ... with m = n // 2."""
    m = n // 2
    order = [m]
    for d in range(1, n + 1):
        for cand in (m - d, m + d):
            if 0 <= cand < n:
                order.append(cand)
    return order[:n]


def select_probe_rows(labels: np.ndarray, C: int, M: int):
    """Probe rows and weights shared by all heads: (probe_idx [M] int, weights [M] float64)."""
    labels = np.asarray(labels)
    S = labels.size
    if not 0 < M <= S:
        raise ValueError("need 0 < M <= S")
    members = [np.nonzero(labels == a)[0] for a in range(C)]
    queues = [[int(mem[j]) for j in middle_out(len(mem))] for mem in members]
    nonempty = [a for a in range(C) if len(members[a]) > 0]
    n_ne = len(nonempty)
    taken, taken_from = [], []
    first_round = (nonempty if M >= n_ne
                   else [nonempty[int(np.floor((j + 0.5) * n_ne / M))] for j in range(M)])
    cursor = [0] * C
    visit = first_round
    while len(taken) < M:
        for a in visit:
            if len(taken) == M:
                break
            if cursor[a] < len(queues[a]):
                taken.append(queues[a][cursor[a]])
                taken_from.append(a)
                cursor[a] += 1
        visit = nonempty
    taken_from = np.array(taken_from)
    per_cluster = np.bincount(taken_from, minlength=C)
    sizes = np.array([len(m) for m in members])
    w = sizes[taken_from] / per_cluster[taken_from]
    return np.array(taken, dtype=np.int64), w / w.sum()


def ridge_fit(o_sparse_p: np.ndarray, o_dense_p: np.ndarray, weights: np.ndarray, lam: float,
              rank: int) -> dict:
    """Fit the correction from probe rows; returns the fitted pieces and the folded map.

    o_sparse_p, o_dense_p: [M, D] sparse and exact outputs of the probe rows.
    Returns a dict with mu, sigma [D], W [D, D], rbar [D], P [D, D], r_eff, and the folded
    affine map A [D, D], c [D] such that the correction of a row o is  o @ A + c.
    """
    xs = np.asarray(o_sparse_p, dtype=np.float64)
    xd = np.asarray(o_dense_p, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    w = w / w.sum()
    D = xs.shape[1]
    R = xd - xs
    # Weighted standardization of the sparse output.
    mu = w @ xs
    sigma = np.sqrt(w @ (xs - mu) ** 2)
    sigma = np.where(sigma < 1e-6, 1.0, sigma)
    X = (xs - mu) / sigma
    # Unpenalized intercept: the weighted mean residual.
    rbar = w @ R
    Rc = R - rbar
    # Weighted ridge: (X^T Omega X + lambda I) W = X^T Omega Rc, by Cholesky.
    G = X.T @ (w[:, None] * X) + lam * np.eye(D)
    W = scipy.linalg.cho_solve(scipy.linalg.cho_factor(G, lower=True), X.T @ (w[:, None] * Rc))
    # Principal residual directions: top eigenvectors of Rc^T Omega Rc.
    CR = Rc.T @ (w[:, None] * Rc)
    evals, evecs = np.linalg.eigh(CR)
    evals, evecs = evals[::-1], evecs[:, ::-1]
    if evals[0] > 0:
        r_eff = int(min(rank, np.count_nonzero(evals > 1e-12 * evals[0])))
    else:
        r_eff = 0
    Vr = evecs[:, :r_eff]
    P = Vr @ Vr.T
    A = (W / sigma[:, None]) @ P
    c = rbar - mu @ A
    return dict(mu=mu, sigma=sigma, W=W, rbar=rbar, P=P, r_eff=r_eff, A=A, c=c, X=X, Rc=Rc,
                evals=evals)


def correction(o: np.ndarray, fit: dict) -> np.ndarray:
    """The correction of rows o, written in the fitted pieces: ((o - mu)/sigma) W P + rbar."""
    o = np.asarray(o, dtype=np.float64)
    return ((o - fit["mu"]) / fit["sigma"]) @ fit["W"] @ fit["P"] + fit["rbar"]


def apply_correction(o: np.ndarray, A: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Repaired rows: o + o @ A + c, for every row given."""
    o = np.asarray(o, dtype=np.float64)
    return o + o @ A + c
