"""Pins for the oracle's error-aware routing (CPU only).

The pages print no worked example for the router, so the oracle is pinned by what the
definitions fix: query centroids of ramps in
closed form; zero compensation error where a centroid is exact (identical keys and values,
one-key clusters); the exact identity between the first-order error and the brute-force
output change of compensating one block, (O' - O)(1 + z_hat - Z_c) = delta, with O' from a
softmax over the modified key set written out as a loop; invariance under reordering keys
inside a cluster; and hand-worked routes.  The near-tie exclusion that the GPU route
parity uses (a test helper, not part of the oracle) is pinned on hand-worked rows here too.
"""

import numpy as np
import pytest
import torch

from oracle import routing as ort


def test_query_centroids_ramp_and_empty_cluster():
    B, H, S, D = 1, 2, 12, 3
    i = np.arange(S)[None, None, :, None]
    q = (i + 10.0 * np.arange(H)[None, :, None, None] + 100.0 * np.arange(D)) * np.ones((B, H, S, D))
    lab = np.array([0, 0, 0, 2, 2, 0, 2, 2, 2, 0, 0, 2])  # cluster 1 empty
    qb = ort.query_centroids(q, lab, 3)
    for h in range(H):
        for c, rows in ((0, [0, 1, 2, 5, 9, 10]), (2, [3, 4, 6, 7, 8, 11])):
            np.testing.assert_allclose(qb[0, h, c], np.mean(rows) + 10.0 * h + 100.0 * np.arange(D), rtol=1e-15)
        assert np.all(qb[0, h, 1] == 0.0)


def _setup(seed, S=40, D=6, C=5, Cq=3, H=2, Hkv=1):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, Hkv, S, D))
    v = rng.standard_normal((1, Hkv, S, D))
    klab = rng.integers(0, C, S)
    qbar = rng.standard_normal((1, H, Cq, D))
    return qbar, k, v, klab


def test_exact_centroids_have_zero_error():
    qbar, k, v, klab = _setup(1)
    # cluster 2: every key and value identical; cluster 4: a single key
    rows2 = np.nonzero(klab == 2)[0]
    k[0, 0, rows2] = k[0, 0, rows2[0]]
    v[0, 0, rows2] = v[0, 0, rows2[0]]
    klab[klab == 4] = 3
    klab[7] = 4
    err = ort.block_compensation_error(qbar, k, v, klab, 5, 0.4)
    assert np.all(np.abs(err[..., 2]) < 1e-15) and np.all(np.abs(err[..., 4]) < 1e-15)
    assert np.all(err[..., [0, 1, 3]] > 1e-6)


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_first_order_error_matches_brute_force_change(seed):
    """Compensate block (a, c) alone, recompute the probe's softmax output by brute force,
    and check (O' - O)(1 + z_hat - Z_c) against delta, whose norm is the error."""
    scale = 0.35
    qbar, k, v, klab = _setup(seed, S=30, D=4, C=4, Cq=2, H=2, Hkv=1)
    err = ort.block_compensation_error(qbar, k, v, klab, 4, scale)
    K, V = k[0, 0], v[0, 0]
    for h in range(2):
        for a in range(2):
            q = qbar[0, h, a]
            logits = [q @ K[j] * scale for j in range(30)]
            mx = max(logits)
            w = [np.exp(x - mx) for x in logits]
            Z = sum(w)
            O = sum(w[j] * V[j] for j in range(30)) / Z
            for c in range(4):
                mem = [j for j in range(30) if klab[j] == c]
                kb = sum(K[j] for j in mem) / len(mem)
                vb = sum(V[j] for j in mem) / len(mem)
                wc = np.exp(q @ kb * scale + np.log(len(mem)) - mx)
                num = sum(w[j] * V[j] for j in range(30) if klab[j] != c) + wc * vb
                den = sum(w[j] for j in range(30) if klab[j] != c) + wc
                O2 = num / den
                Zc = sum(w[j] for j in mem) / Z
                zhat = wc / Z
                lhs = (O2 - O) * (1.0 + zhat - Zc)
                assert abs(np.linalg.norm(lhs) - err[0, h, a, c]) < 1e-12 * max(1.0, err[0, h, a, c])


def test_error_invariant_to_key_order_inside_clusters():
    qbar, k, v, klab = _setup(5)
    err = ort.block_compensation_error(qbar, k, v, klab, 5, 0.3)
    perm = np.random.default_rng(6).permutation(klab.size)
    err2 = ort.block_compensation_error(qbar, k[:, :, perm], v[:, :, perm], klab[perm], 5, 0.3)
    np.testing.assert_allclose(err, err2, rtol=1e-12, atol=1e-15)


def test_gqa_heads_share_kv():
    qbar, k, v, klab = _setup(7, H=4, Hkv=2)
    err = ort.block_compensation_error(qbar, k, v, klab, 5, 0.3)
    one = ort.block_compensation_error(qbar[:, 2:4], k[:, 1:2], v[:, 1:2], klab, 5, 0.3)
    np.testing.assert_array_equal(err[:, 2:4], one)


def test_route_hand_worked():
    # counts 10, 20, 0, 5, 30; errors give ratios 0.5, 0.5, -, 2.0, 0.1
    n = np.array([10, 20, 0, 5, 30])
    err = np.array([[[[5.0, 10.0, 7.0, 10.0, 3.0]]]])
    keep = lambda budget: ort.error_aware_route(err, n, budget)[0, 0, 0].tolist()
    assert keep(0) == [0, 0, 0, 1, 0]         # at least one cluster: the best ratio
    assert keep(5) == [0, 0, 0, 1, 0]         # budget reached exactly
    assert keep(6) == [1, 0, 0, 1, 0]         # tie 0.5 / 0.5: the lower index first
    assert keep(15) == [1, 0, 0, 1, 0]
    assert keep(16) == [1, 1, 0, 1, 0]
    assert keep(36) == [1, 1, 0, 1, 1]
    assert keep(10 ** 9) == [1, 1, 0, 1, 1]   # an empty cluster is never kept


def test_route_rows_independent():
    n = np.array([4, 4, 4])
    err = np.array([[[[1.0, 2.0, 3.0], [3.0, 2.0, 1.0]], [[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]]]])
    keep = ort.error_aware_route(err, n, 8)
    assert keep[0, 0].tolist() == [[0, 1, 1], [1, 1, 0]]
    assert keep[0, 1].tolist() == [[1, 1, 0], [1, 1, 0]]


def test_route_float64_ratios():
    """1 / 3 and the float32 nearest to 1/3 are distinct float64 quotients: the larger one
    wins in float64 (a float32 evaluation would tie them and take the lower index)."""
    n = np.array([3, 1])
    third = float(np.float32(1.0) / np.float32(3.0))
    err = np.array([[[[1.0, third]]]])
    assert third > 1.0 / 3.0
    assert ort.error_aware_route(err, n, 1)[0, 0, 0].tolist() == [0, 1]


def test_route_fragile_rows_helper():
    """The GPU route comparison skips rows whose cut falls inside a run of float64 ratios that
    are near-tied but not all equal (a float32 quotient can tie them and order them by index):
    hand-worked rows."""
    from gpu_common import round_bf16, route_fragile_rows

    n = np.array([3, 1, 2, 4])
    third = float(np.float32(1.0) / np.float32(3.0))
    # ratios 1/3, third, 0.25, 0.5: cut after one cluster (budget 1) lands on ratio 0.5 (alone) -> fine
    err = np.array([[[[1.0, third, 0.5, 2.0]]]])
    assert not route_fragile_rows(err, n, 1)[0, 0, 0]
    # budget 5: 0.5 (4 keys), then third (1 key): the cut at third, near-tied with 1/3 -> fragile
    assert route_fragile_rows(err, n, 5)[0, 0, 0]
    # exact ties only (0.5 and 0.5) at the cut: both sides order them by index -> not fragile
    err2 = np.array([[[[1.5, 0.5, 1.0, 2.0]]]])
    assert not route_fragile_rows(err2, n, 5)[0, 0, 0]
    # bfloat16 rounding helper: torch's conversion, ties to even
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000),
                        [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x), want)
    assert round_bf16([1.0 + 2 ** -8])[0] == 1.0
    assert round_bf16([1.0 + 3 * 2 ** -8])[0] == 1.0 + 2 ** -6
