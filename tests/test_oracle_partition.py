"""Pins for the oracle's response-coupled partitioning (CPU only).

The pages print no worked example, so the oracle is pinned by hand-worked k-means runs (a
1-D run to convergence, a tie between centres, a centre left without points), properties any
k-means has (well-separated blobs are recovered whatever the dimension order, scale or offset
of the data; the final labels are nearest centres), hand-worked sampled queries and response
profiles, and an end-to-end case whose keys and queries come from separated response groups.
"""

import numpy as np
import pytest

from oracle import partition as op


def test_evenly_spaced():
    assert op.evenly_spaced(5, 2).tolist() == [1, 3]
    assert op.evenly_spaced(5, 3).tolist() == [0, 2, 4]
    assert op.evenly_spaced(32760, 48)[[0, -1]].tolist() == [341, 32418]


def test_kmeans_hand_worked_1d():
    # centres start at x[1] = 1 and x[3] = 11; the first assignment puts 10, 11, 20 with 11,
    # the means become 0.5 and 41/3, and the next assignment is the same: converged
    X = np.array([[0.0], [1.0], [10.0], [11.0], [20.0]])
    labels, centres = op.kmeans(X, 2, iters=4)
    assert labels.tolist() == [0, 0, 1, 1, 1]
    np.testing.assert_allclose(centres[:, 0], [0.5, 41.0 / 3.0], rtol=0, atol=1e-15)


def test_kmeans_tie_and_empty_centre():
    # centres start at x[0] = 0, x[2] = 0, x[4] = 5: the zeros tie between centres 0 and 1 and
    # go to 0; centre 1 gets no point and stays at 0
    X = np.array([[0.0], [0.0], [0.0], [0.0], [5.0]])
    labels, centres = op.kmeans(X, 3, iters=2)
    assert labels.tolist() == [0, 0, 0, 0, 2]
    assert centres[:, 0].tolist() == [0.0, 0.0, 5.0]


def _blobs(seed, n_per, C, F, sep=50.0):
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((C, F)) * sep
    truth = np.repeat(np.arange(C), n_per)
    X = centres[truth] + rng.standard_normal((C * n_per, F))
    perm = rng.permutation(X.shape[0])
    return X[perm], truth[perm]


def _same_partition(a, b):
    """Labelings a and b define the same groups (up to the names of the groups)."""
    pairs = set(zip(a.tolist(), b.tolist()))
    return len(pairs) == len(set(a.tolist())) == len(set(b.tolist()))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kmeans_recovers_separated_blobs_and_is_invariant(seed):
    X, truth = _blobs(seed, 30, 5, 7)
    # deterministic starts can land two centres in one blob; give each blob a start by ordering
    # the points so that the evenly spaced positions hit distinct blobs
    order = np.argsort(truth, kind="stable")
    X, truth = X[order], truth[order]
    labels, centres = op.kmeans(X, 5)
    assert _same_partition(labels, truth)
    # the final labels are nearest centres of the final centres
    d = op.sq_distances(X, centres)
    assert np.all(d[np.arange(X.shape[0]), labels] <= d.min(axis=1))
    # the same partition after permuting the dimensions, scaling and shifting the data
    pf = np.random.default_rng(seed).permutation(X.shape[1])
    for Y in (X[:, pf], 3.5 * X, X + 100.0):
        assert np.array_equal(op.kmeans(Y, 5)[0], labels)


def test_sampled_queries_round_robin_over_heads():
    G, S, D = 2, 8, 3
    q = np.arange(G * S * D, dtype=np.float64).reshape(G, S, D)
    qs = op.sampled_queries(q, rK=4)  # positions 1, 3, 5, 7 from heads 0, 1, 0, 1
    assert np.array_equal(qs, np.stack([q[0, 1], q[1, 3], q[0, 5], q[1, 7]]))


def test_key_features_hand_worked():
    k = np.array([[1.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    qs = np.array([[2.0, 1.0], [0.0, -1.0]])
    # responses: key 0 -> (2, 0), key 1 -> (2, -2), key 2 -> (3, -1), times the scale 0.5
    np.testing.assert_allclose(op.key_features(k, qs, 0.5), [[1.0, 0.0], [1.0, -1.0], [1.5, -0.5]])


def test_query_coordinates_hand_worked():
    # two key groups with centroids (1, 0) and (0, 2); a group's query is its heads' mean
    k = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 2.0]])
    k_labels = np.array([0, 0, 1])
    q = np.array([[[3.0, 4.0], [0.0, 0.0]], [[1.0, 0.0], [0.0, 0.0]]])  # [G=2, S=2, D=2]
    g = op.query_coordinates(q, k, k_labels, 2, 1.0, rQ=64)
    # token 0: mean query (2, 2) -> responses (2, 4) -> unit (1, 2)/sqrt(5); token 1: zero
    np.testing.assert_allclose(g[0], np.array([1.0, 2.0]) / np.sqrt(5.0), atol=1e-15)
    assert np.all(g[1] == 0.0)
    # rQ below the group count takes evenly spaced groups
    k8 = np.eye(8)
    g8 = op.query_coordinates(np.ones((1, 3, 8)), k8, np.arange(8), 8, 1.0, rQ=2)
    assert g8.shape == (3, 2)  # groups 2 and 6


def test_partition_separates_response_groups():
    """Keys in 4 directions, queries aligned with them: the keys split by direction, and the
    queries by the key group they respond to."""
    rng = np.random.default_rng(7)
    D, S, C = 16, 400, 4
    dirs = np.linalg.qr(rng.standard_normal((D, D)))[0][:C] * 6.0
    kt = np.repeat(np.arange(C), S // C)
    # (the evenly spaced starting points fall in distinct groups: tokens 50, 150, 250, 350)
    qt = (np.repeat(np.arange(C), S // C) + 1) % C
    k = dirs[kt] + 0.05 * rng.standard_normal((S, D))
    q = (dirs[qt] + 0.05 * rng.standard_normal((S, D)))[None]
    kl, ql = op.response_coupled_partition(q, k, C, C, 0.25, rK=48, rQ=64)
    assert _same_partition(kl, kt) and _same_partition(ql, qt)
    assert kl.dtype == np.int32 and ql.dtype == np.int32
