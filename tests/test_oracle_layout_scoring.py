"""Pins for the oracle's layout, centroid, scoring and top-p stages (CPU only).

Each test checks the oracle against something other than itself: hand-worked fixtures in
tests/golden/, a pure-Python brute force of the page's literal description, a textbook
softmax from SciPy, or an invariant the definition implies.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import centroids as oc
from oracle import layout as ol
from oracle import scoring as osc
from oracle import topp as otp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- layout


def test_layout_golden():
    g = golden("layout_tiny.json")
    perm, offsets, counts = ol.cluster_layout(np.array(g["labels"]), g["C"])
    assert perm.tolist() == g["perm"]
    assert offsets.tolist() == g["offsets"]
    assert counts.tolist() == g["counts"]


def test_layout_properties_random():
    rng = np.random.default_rng(0)
    for _ in range(20):
        S, C = int(rng.integers(1, 300)), int(rng.integers(1, 40))
        labels = rng.integers(0, C, size=S)
        perm, offsets, counts = ol.cluster_layout(labels, C)
        assert sorted(perm.tolist()) == list(range(S))
        lp = labels[perm]
        assert np.all(np.diff(lp) >= 0)
        for c in range(C):
            run = perm[offsets[c]:offsets[c + 1]]
            assert np.all(labels[run] == c)
            assert np.all(np.diff(run) > 0)  # stable: original order inside a cluster
            assert counts[c] == np.count_nonzero(labels == c)


def test_layout_rejects_bad_labels():
    with pytest.raises(ValueError):
        ol.cluster_layout(np.array([0, 3]), 3)


def test_tile_labels_golden():
    g = golden("tile_labels_tiny.json")
    lab = ol.tile_labels(g["T"], g["H"], g["W"], tuple(g["tile"]), 0)
    assert lab.tolist() == g["labels_tile"]
    lab = ol.tile_labels(g["T"], g["H"], g["W"], tuple(g["tile"]), g["chunk"])
    assert lab.tolist() == g["labels_chunk"]


def test_tile_labels_chunked_clusters_are_tiles_when_tiles_divide():
    # When tiles divide the grid and hold exactly `chunk` tokens, chunked labels equal
    # the tile ids.
    tile = (2, 4, 4)
    a = ol.tile_labels(4, 8, 8, tile, 0)
    b = ol.tile_labels(4, 8, 8, tile, 32)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- centroids


def test_centroids_hand_and_identical_keys():
    k = np.array([[1.0, 3.0], [5.0, 5.0], [3.0, 5.0], [7.0, 7.0]])
    v = np.array([[0.0, 1.0], [1.0, 1.0], [2.0, 3.0], [4.0, 4.0]])
    labels = np.array([0, 2, 0, 2])
    kbar, vbar, n = oc.centroids(k, v, labels, 3)
    assert n.tolist() == [2, 0, 2]
    assert np.allclose(kbar[0], [2.0, 4.0]) and np.allclose(kbar[2], [6.0, 6.0])
    assert np.allclose(vbar[0], [1.0, 2.0]) and np.allclose(vbar[2], [2.5, 2.5])
    assert np.all(kbar[1] == 0) and np.all(vbar[1] == 0)
    # identical keys in a cluster: the centroid is that key
    rng = np.random.default_rng(1)
    base = rng.standard_normal((4, 8))
    labels = rng.integers(0, 4, size=50)
    kbar, _, _ = oc.centroids(base[labels], rng.standard_normal((50, 8)), labels, 4)
    present = np.bincount(labels, minlength=4) > 0
    assert np.allclose(kbar[present], base[present], atol=1e-14)


def test_centroids_permutation_invariant():
    rng = np.random.default_rng(2)
    k, v = rng.standard_normal((60, 5)), rng.standard_normal((60, 5))
    labels = rng.integers(0, 6, size=60)
    p = rng.permutation(60)
    a = oc.centroids(k, v, labels, 6)
    b = oc.centroids(k[p], v[p], labels[p], 6)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-13)


# ---------------------------------------------------------------- scoring


def test_scores_golden_orientation_and_padding():
    g = golden("antidiag_tiny.json")
    q = np.array(g["q"], dtype=float)[:, None]
    k = np.array(g["k"], dtype=float)[:, None]
    s = osc.antidiagonal_block_scores(q, k, None, g["block"], g["stride"], g["score_scale"])
    assert np.allclose(s, g["scores"], atol=1e-14)
    q = np.array(g["q_pad"], dtype=float)[:, None]
    k = np.array(g["k_pad"], dtype=float)[:, None]
    s = osc.antidiagonal_block_scores(q, k, None, g["block"], g["stride"], g["score_scale"])
    assert np.allclose(s, g["scores_pad"], atol=1e-14)


def brute_scores(q, k, block, stride, sigma):
    """The page's description, literally: zero-pad, take every stride x stride sub-block of
    q k^T, sum its anti-diagonal, softmax each strided row, sum block x block tiles,
    normalize rows.  Pure Python loops."""
    S, D = q.shape
    nb = -(-S // block)
    n = nb * block
    qp = np.zeros((n, D))
    kp = np.zeros((n, D))
    qp[:S], kp[:S] = q, k
    ns = n // stride
    full = qp @ kp.T
    logit = np.zeros((ns, ns))
    for i in range(ns):
        for j in range(ns):
            sub = full[i * stride:(i + 1) * stride, j * stride:(j + 1) * stride]
            logit[i, j] = sigma * sum(sub[r, stride - 1 - r] for r in range(stride))
    p = scipy.special.softmax(logit, axis=1)
    r = block // stride
    mass = np.zeros((nb, nb))
    for a in range(nb):
        for c in range(nb):
            mass[a, c] = p[a * r:(a + 1) * r, c * r:(c + 1) * r].sum()
    return mass / mass.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("S,D,block,stride", [(32, 3, 8, 4), (30, 4, 8, 2), (45, 2, 9, 3), (16, 5, 4, 4)])
def test_scores_match_bruteforce(S, D, block, stride):
    rng = np.random.default_rng(S * 7 + D)
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    s = osc.antidiagonal_block_scores(q, k, None, block, stride, 0.7)
    assert np.allclose(s, brute_scores(q, k, block, stride, 0.7), atol=1e-13)


def test_stride_one_is_block_mass_of_dense_softmax():
    rng = np.random.default_rng(3)
    S, D, b = 48, 6, 8
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    sig = 1 / math.sqrt(D)
    p = scipy.special.softmax(sig * q @ k.T, axis=1)
    want = p.reshape(S // b, b, S // b, b).sum(axis=(1, 3)) / b
    got = osc.antidiagonal_block_scores(q, k, None, b, 1, sig)
    assert np.allclose(got, want, atol=1e-14)


def test_scores_rows_sum_to_one_and_perm_gathers():
    rng = np.random.default_rng(4)
    S, D = 64, 8
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    perm = rng.permutation(S)
    s = osc.antidiagonal_block_scores(q, k, perm, 16, 4, 0.3)
    assert np.allclose(s.sum(axis=1), 1.0, atol=1e-14)
    s2 = osc.antidiagonal_block_scores(q[perm], k[perm], None, 16, 4, 0.3)
    assert np.allclose(s, s2, atol=1e-15)


def test_scores_key_block_permutation_equivariance():
    rng = np.random.default_rng(5)
    S, D, b = 64, 4, 16
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    bp = np.array([2, 0, 3, 1])
    kperm = np.concatenate([np.arange(c * b, (c + 1) * b) for c in bp])
    s = osc.antidiagonal_block_scores(q, k, None, b, 4, 0.5)
    s2 = osc.antidiagonal_block_scores(q, k[kperm], None, b, 4, 0.5)
    assert np.allclose(s2, s[:, bp], atol=1e-14)


def test_pooled_scores_mean():
    x = np.arange(2 * 3 * 2 * 2, dtype=float).reshape(6, 2, 2)
    p = osc.pooled_group_scores(x, 3)
    assert p.shape == (2, 2, 2)
    assert np.allclose(p[0], (x[0] + x[1] + x[2]) / 3)


# ---------------------------------------------------------------- top-p


def test_topp_golden():
    g = golden("topp_tiny.json")
    for case in g["cases"]:
        assert otp.top_p_row(np.array(g["row"]), case["tau"]).tolist() == case["keep"]
    assert otp.top_p_row(np.array(g["row_block0_small"]), g["tau_block0_small"]).tolist() == g["keep_block0_small"]


def test_fragile_blocks_golden():
    """Hand-worked rows for the mask-parity exclusion: near-mass blocks on both sides of tau,
    near-ties straddling the cut (two and three blocks), a near-tie inside the kept set and
    ties just outside the window, which must not be excluded."""
    g = golden("fragile_blocks_tiny.json")
    for case in g["cases"]:
        row = np.array(case["row"])
        assert otp.top_p_row(row, case["tau"]).tolist() == case["keep"], case["name"]
        got = otp.fragile_blocks(row, case["tau"]).astype(int).tolist()
        assert got == case["fragile"], (case["name"], got)
    # Permuting the blocks permutes the exclusion (the definition does not depend on position).
    for case in g["cases"]:
        row = np.array(case["row"])
        p = np.arange(row.size)[::-1]
        assert np.array_equal(otp.fragile_blocks(row[p], case["tau"]), np.array(case["fragile"], bool)[p]), case["name"]


def brute_topp(row, tau):
    """All subsets: minimum cardinality with mass >= tau * total; among those the largest
    mass; remaining ties by lexicographically smallest sorted index tuple."""
    n = len(row)
    total = sum(row)
    for size in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            m = sum(row[i] for i in sub)
            if m >= tau * total:
                key = (-m, sub)
                if best is None or key < best[0]:
                    best = (key, sub)
        if best is not None:
            keep = np.zeros(n, dtype=np.uint8)
            keep[list(best[1])] = 1
            return keep
    return np.ones(n, dtype=np.uint8)


def test_topp_matches_bruteforce():
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        row = rng.dirichlet(np.full(n, 0.5))
        tau = float(rng.uniform(0.05, 0.99))
        keep = otp.top_p_row(row, tau)
        excl = otp.fragile_blocks(row, tau, 1e-12, 0.0)
        bf = brute_topp(row, tau)
        assert np.array_equal(keep[~excl], bf[~excl]), (row, tau)
        assert keep.sum() >= 1


def test_topp_tiny_tau_keeps_argmax_and_scale_invariance():
    rng = np.random.default_rng(7)
    for _ in range(50):
        row = rng.uniform(size=12)
        keep = otp.top_p_row(row, 1e-9)
        assert keep.sum() == 1 and keep[np.argmax(row)] == 1
        tau = float(rng.uniform(0.1, 0.95))
        assert np.array_equal(otp.top_p_row(row, tau), otp.top_p_row(row * 37.5, tau))


def test_topp_per_head_tau_and_lists():
    scores = np.array([[[0.7, 0.2, 0.1]], [[0.7, 0.2, 0.1]]])
    keep = otp.top_p_block_mask(scores, np.array([0.6, 0.85]))
    assert keep[0, 0].tolist() == [1, 0, 0] and keep[1, 0].tolist() == [1, 1, 0]
    counts, idx = otp.kept_lists(keep)
    assert counts.tolist() == [1, 2] and idx[1].tolist() == [0, 1]
