"""GPU parity of response-coupled partitioning (bsa_kmeans, bsa_response_partition) against the
oracle ("Partition the Support, Reconstruct the Residual", Response-Coupled Partitioning).

The kernels take the nearest centre from |c|^2 - 2 x.c with x.c as split-bfloat16 products
(x = hi + lo in bfloat16, hi.hi + hi.lo + lo.hi summed in float32: within about 3e-5 |x| |c|),
the oracle from float64 squared differences, so a point whose two nearest centres are closer
than that rounding may go either way.  Every comparison therefore checks what is
unique exactly and the rest for validity: labels equal the oracle's wherever the oracle's
best centre wins by more than the rounding bound; every label is a nearest centre (within the
bound) of the centres it is returned with; centres are the means of the points they were
moved to.  On data with separated groups (no near ties anywhere) the whole result is exact.
"""

import numpy as np
import pytest
import torch

from oracle import partition as op
from synthetic import make_config, make_custom

from gpu_common import dev, say

pytestmark = pytest.mark.gpu

F = 64  # stored feature width


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _pad(X: np.ndarray) -> np.ndarray:
    out = np.zeros(X.shape[:-1] + (F,), dtype=np.float32)
    out[..., :X.shape[-1]] = X
    return out


def _bound(X: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Per-point bound on the rounding of |c|^2 - 2 x.c, [N]: 2e-5 (|x| + |c|)^2 >= 8e-5 |x| |c|,
    above the split-bfloat16 products' 2 * (3 * 2^-18 + 64 * 2^-24) |x| |c| ~ 3e-5 |x| |c|."""
    xn = (X * X).sum(axis=1)
    cn = (centres * centres).sum(axis=1).max()
    return 2e-5 * (xn + cn + 2.0 * np.sqrt(xn * cn)) + 1e-30


def check_nearest(X: np.ndarray, centres: np.ndarray, labels: np.ndarray, what: str) -> None:
    """Every label is a nearest centre within the rounding bound (float64 distances)."""
    d = op.sq_distances(X, centres)
    got = d[np.arange(X.shape[0]), labels]
    slack = got - d.min(axis=1)
    bad = slack > _bound(X, centres)
    assert not bad.any(), f"{what}: {bad.sum()} labels are not nearest centres (worst slack {slack.max():.3e})"


def clear_rows(X: np.ndarray, centres: np.ndarray) -> np.ndarray:
    """Points whose nearest centre wins by more than the rounding bound."""
    d = op.sq_distances(X, centres)
    two = np.partition(d, 1, axis=1)[:, :2] if centres.shape[0] > 1 else np.c_[d, d + np.inf]
    return (two[:, 1] - two[:, 0]) > _bound(X, centres)


# ------------------------------------------------------------------ k-means


@pytest.mark.parametrize("P,N,nf,C,seed", [(3, 3000, 48, 100, 0), (2, 5000, 64, 300, 1), (1, 777, 16, 5, 2),
                                           (2, 1, 7, 1, 3), (1, 9000, 33, 4000, 4)])
def test_kmeans_first_assignment_matches_oracle(bsa, P, N, nf, C, seed):
    """iters = 0: the starting centres are the evenly spaced points, the labels their nearest
    centres -- equal to the oracle's outside near ties."""
    say(f"kmeans assign P={P} N={N} nf={nf} C={C}")
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((P, N, nf)).astype(np.float32)
    labels, centres = bsa.kmeans(torch.from_numpy(_pad(X)).cuda(), C, iters=0, nf=nf)
    labels, centres = labels.cpu().numpy(), centres.cpu().numpy()
    for p in range(P):
        X64 = X[p].astype(np.float64)
        start = X64[op.evenly_spaced(N, C)]
        assert np.array_equal(centres[p, :, :nf], start) and not centres[p, :, nf:].any()
        ref = op.nearest_centre(X64, start)
        clear = clear_rows(X64, start)
        assert clear.mean() > 0.99
        assert np.array_equal(labels[p][clear], ref[clear]), f"p={p}: {np.sum(labels[p][clear] != ref[clear])} differ"
        check_nearest(X64, start, labels[p], f"p={p}")


@pytest.mark.parametrize("P,N,nf,C,seed", [(2, 4000, 48, 64, 5), (1, 2500, 64, 700, 6)])
def test_kmeans_lloyd_steps(bsa, P, N, nf, C, seed):
    """One Lloyd step on any data: the centres after iters = 1 are the means of the points of
    the first assignment (a centre without points stays at its start), and the last labels
    are nearest centres of them."""
    say(f"kmeans lloyd P={P} N={N} nf={nf} C={C}")
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((P, N, nf)) * 3.0 + 1.0).astype(np.float32)
    x = torch.from_numpy(_pad(X)).cuda()
    l0 = bsa.kmeans(x, C, iters=0, nf=nf)[0].cpu().numpy()
    l1, c1 = (t.cpu().numpy() for t in bsa.kmeans(x, C, iters=1, nf=nf))
    for p in range(P):
        X64 = X[p].astype(np.float64)
        start = X64[op.evenly_spaced(N, C)]
        want = op.centre_means(X64, l0[p].astype(np.int64), start)
        np.testing.assert_allclose(c1[p, :, :nf], want, rtol=1e-5, atol=1e-5 * np.abs(X64).max())
        check_nearest(X64, c1[p, :, :nf].astype(np.float64), l1[p], f"p={p}")


def _blobs(rng, P, C, n_per, nf, sep=40.0):
    """Separated blobs; the points are ordered by blob so that the evenly spaced starting
    points fall in distinct blobs."""
    X = np.empty((P, C * n_per, nf), dtype=np.float32)
    truth = np.repeat(np.arange(C), n_per)
    for p in range(P):
        centres = rng.standard_normal((C, nf)) * sep
        X[p] = centres[truth] + rng.standard_normal((C * n_per, nf))
    return X


def test_kmeans_separated_blobs_exact(bsa):
    say("kmeans blobs")
    rng = np.random.default_rng(8)
    P, C, n_per, nf = 3, 40, 50, 48
    X = _blobs(rng, P, C, n_per, nf)
    labels, centres = (t.cpu().numpy() for t in bsa.kmeans(torch.from_numpy(_pad(X)).cuda(), C, iters=4, nf=nf))
    for p in range(P):
        ref_l, ref_c = op.kmeans(X[p].astype(np.float64), C, 4)
        assert np.array_equal(labels[p], ref_l)
        np.testing.assert_allclose(centres[p, :, :nf], ref_c, rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------ the whole partition


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_response_partition_separated_groups_exact(bsa, dtype, D):
    """Keys in Ck directions, queries aligned with them (two query heads sharing the keys):
    both partitions equal the oracle's label for label."""
    say(f"response partition separated {dtype} D={D}")
    rng = np.random.default_rng(9)
    B, Hkv, G, S, C = 2, 2, 2, 2048, 8
    q = np.empty((B, Hkv * G, S, D))
    k = np.empty((B, Hkv, S, D))
    for b in range(B):
        for h in range(Hkv):
            dirs = np.linalg.qr(rng.standard_normal((D, D)))[0][:C] * 6.0
            kt = np.repeat(np.arange(C), S // C)
            qt = (kt + 1) % C
            k[b, h] = dirs[kt] + 0.05 * rng.standard_normal((S, D))
            for g in range(G):
                q[b, h * G + g] = dirs[qt] + 0.05 * rng.standard_normal((S, D))
    qd, kd = dev(q, dtype), dev(k, dtype)
    q = qd.float().cpu().numpy().astype(np.float64)  # the rounded values both sides read
    k = kd.float().cpu().numpy().astype(np.float64)
    kl, ql = (t.cpu().numpy() for t in bsa.response_partition(qd, kd, C, C, scale=0.25))
    for b in range(B):
        for h in range(Hkv):
            rk, rq = op.response_coupled_partition(q[b, h * G:(h + 1) * G], k[b, h], C, C, 0.25)
            assert np.array_equal(kl[b, h], rk) and np.array_equal(ql[b, h], rq), f"b={b} h={h}"


def _validate_partition(q, k, kl, ql, kc, qc, Cq, Ck, scale, what):
    """Labels valid for the oracle's features: key labels nearest (within rounding) to the
    returned key centres in the oracle's key-profile space; query labels nearest to the
    returned query centres in the oracle's query coordinates built from the returned key
    labels; every group index in range.  Returns the fraction of clear rows that equal the
    oracle's own partition of the same inputs."""
    assert kl.min() >= 0 and kl.max() < Ck and ql.min() >= 0 and ql.max() < Cq
    kf = op.key_features(k, op.sampled_queries(q), scale)
    check_nearest(kf, kc[:, :op.RK].astype(np.float64), kl, f"{what} keys")
    qf = op.query_coordinates(q, k, kl, Ck, scale)
    check_nearest(qf, qc[:, :qf.shape[1]].astype(np.float64), ql, f"{what} queries")
    assert not kc[:, op.RK:].any() and not qc[:, qf.shape[1]:].any()


@pytest.mark.parametrize("case", ["custom_gqa", "video_head"])
def test_response_partition_valid(bsa, case):
    """Workload-shaped inputs (near ties happen): every label is valid for the oracle's
    features and the returned centres."""
    if case == "custom_gqa":
        wl = make_custom(12, B=2, Hq=4, Hkv=2, S=3000, D=128, dtype="bf16")
        Cq, Ck = 24, 24
    else:
        wl = make_config(2, heads=[7])  # one head of the video workload, full sequence
        Cq, Ck = 256, 256
    say(f"response partition valid {case} S={wl.S} Cq={Cq} Ck={Ck}")
    qd, kd = dev(wl.q, wl.dtype), dev(wl.k, wl.dtype)
    kl, ql, kc, qc = (t.cpu().numpy() for t in bsa.response_partition(qd, kd, Cq, Ck, scale=wl.scale,
                                                                       return_centres=True))
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        for h in range(wl.Hkv):
            _validate_partition(wl.q[b, h * G:(h + 1) * G], wl.k[b, h], kl[b, h], ql[b, h], kc[b, h], qc[b, h],
                                Cq, Ck, wl.scale, f"b={b} h={h}")


def test_response_partition_rejects(bsa):
    q = torch.zeros(1, 2, 100, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception):
        bsa.response_partition(q, k, 101, 4)  # more groups than tokens
    with pytest.raises(Exception):
        bsa.response_partition(q, k, 4, 4, rK=65)
    with pytest.raises(Exception):
        bsa.response_partition(q[:, :, :, :32].contiguous(), k[:, :, :, :32].contiguous(), 4, 4)
