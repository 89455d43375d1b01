"""Response-coupled partitioning (oracle; test infrastructure only).

Page: "Partition the Support, Reconstruct the Residual" (summary page), the paragraph on
Response-Coupled Partitioning: queries are sampled from the current call; keys are grouped
by their pre-softmax responses to those queries, so keys with similar response profiles share
a K/V block and values follow their keys; the centroids of those key groups then give the
query coordinates, so that queries with similar response direction share a route; one
asymmetric pass (keys, then queries; no alternating refinement); feature ranks rK = 48 and
rQ = 64.  The timing paragraph counts this (online k-means) inside the attention call; the
grouped-query paragraph shares K/V partitions and routes among the query heads of a group.

The pages leave the mechanics open.  Readings (the plainest ones the rest supports):
  * Scope.  One key partition and one query partition per (batch entry, K/V head), shared by
    the group's query heads.
  * Sampled queries.  rK query rows at the evenly spaced token positions
    floor((j + 1/2) S / rK), j < rK, taken round-robin from the group's query heads (head
    j mod G).
  * Key features.  The rK pre-softmax responses of each key, (k . q_s) * scale: the key's
    response profile, an rK-dimensional point (the feature rank rK).
  * Key groups.  k-means (Euclidean) of the key features into Ck groups.
  * Query coordinates.  The responses of each query token to rQ key-group centroids (the
    centroid of a group is the mean of its keys in key space): the groups floor((j + 1/2)
    Ck / rQ), j < min(rQ, Ck); with several query heads the token's query is the mean of its
    heads' queries (the coordinate is linear in the query).  Each coordinate vector is scaled
    to unit length (a response *direction*); a zero vector stays zero.
  * Query groups.  k-means (Euclidean, on the unit vectors) of the query coordinates into Cq
    groups.
  * k-means.  Deterministic Lloyd iterations: the initial centres are the points at the
    evenly spaced positions floor((c + 1/2) N / C); each of `iters` iterations assigns every
    point to its nearest centre (squared distance; equal distances go to the lower centre
    index) and moves every centre to the mean of its points (a centre without points stays
    where it is); a last assignment gives the labels, so every label is a nearest centre of
    the final centres.  iters = 4.
All arithmetic in float64.
"""

from __future__ import annotations

import numpy as np

RK, RQ, ITERS = 48, 64, 4


def evenly_spaced(n_items: int, n_pick: int) -> np.ndarray:
    """Indices floor((j + 1/2) n_items / n_pick), j < n_pick."""
    return ((np.arange(n_pick) + 0.5) * n_items / n_pick).astype(np.int64)


def sq_distances(X: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Squared Euclidean distance of every row of X to every centre, [N, C] (differences
    taken directly, rows in chunks)."""
    out = np.empty((X.shape[0], centres.shape[0]))
    for r0 in range(0, X.shape[0], 512):
        diff = X[r0:r0 + 512, None, :] - centres[None, :, :]
        out[r0:r0 + 512] = (diff * diff).sum(axis=2)
    return out


def nearest_centre(X: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Label of the nearest centre of every row of X (squared Euclidean distance; equal
    distances go to the lower index)."""
    return np.argmin(sq_distances(X, centres), axis=1)  # the first of equal minima


def centre_means(X: np.ndarray, labels: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Mean of each label's rows; a label without rows keeps its old centre."""
    out = centres.copy()
    for c in range(centres.shape[0]):
        rows = labels == c
        if rows.any():
            out[c] = X[rows].mean(axis=0)
    return out


def kmeans(X, C: int, iters: int = ITERS):
    """Deterministic Lloyd k-means (see the header).  Returns (labels [N], centres [C, F])."""
    X = np.asarray(X, dtype=np.float64)
    centres = X[evenly_spaced(X.shape[0], C)].copy()
    for _ in range(iters):
        labels = nearest_centre(X, centres)
        centres = centre_means(X, labels, centres)
    return nearest_centre(X, centres), centres


def sampled_queries(q, rK: int = RK) -> np.ndarray:
    """The rK sampled query rows [rK, D] of a group's query heads q [G, S, D]."""
    q = np.asarray(q, dtype=np.float64)
    G, S, _ = q.shape
    pos = evenly_spaced(S, rK)
    return np.stack([q[j % G, pos[j]] for j in range(rK)])


def key_features(k, qs, scale: float) -> np.ndarray:
    """Response profile of every key: (k . q_s) * scale for the sampled queries, [S, rK]."""
    return (np.asarray(k, dtype=np.float64) @ np.asarray(qs, dtype=np.float64).T) * scale


def query_coordinates(q, k, k_labels, Ck: int, scale: float, rQ: int = RQ) -> np.ndarray:
    """Unit response directions of the query tokens to rQ key-group centroids, [S, rQ']."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qm = q.mean(axis=0)  # the token's query, averaged over the group's heads
    kbar = np.zeros((Ck, k.shape[1]))
    for c in range(Ck):
        rows = k_labels == c
        if rows.any():
            kbar[c] = k[rows].mean(axis=0)
    cols = evenly_spaced(Ck, min(rQ, Ck))
    g = (qm @ kbar[cols].T) * scale
    n = np.sqrt((g * g).sum(axis=1, keepdims=True))
    return np.where(n > 0, g / np.where(n > 0, n, 1.0), 0.0)


def response_coupled_partition(q, k, Cq: int, Ck: int, scale: float, rK: int = RK, rQ: int = RQ,
                               iters: int = ITERS):
    """Key and query labels ([S] each) of one (batch entry, K/V head): q [G, S, D] holds the
    group's query heads, k [S, D] its keys."""
    qs = sampled_queries(q, rK)
    k_labels, _ = kmeans(key_features(k, qs, scale), Ck, iters)
    q_labels, _ = kmeans(query_coordinates(q, k, k_labels, Ck, scale, rQ), Cq, iters)
    return k_labels.astype(np.int32), q_labels.astype(np.int32)
