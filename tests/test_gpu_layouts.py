"""GPU parity with one cluster layout per (batch, K/V head): the partitions of response-coupled
partitioning ("Partition the Support, Reconstruct the Residual", Response-Coupled Partitioning
and grouped-query sharing: K/V partitions and routes are shared by the query heads of a group).

Every stage that reads layouts -- the batched layout itself, the device probe selection, the
packed tiles, the compensated attention, the router's probes, block errors and routes, the
probe rows and the fit -- runs on layouts that differ from head to head, and each head is
checked against the oracle given that head's labels."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import layout as olay
from oracle import repair as orep
from oracle import routing as ort
from synthetic import make_custom

from gpu_common import check_output, dev, host, route_fragile_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def head_labels(seed, P, S, C, lo, hi, empty=True):
    """[P, S] labels: per layout, ragged cluster sizes (some clusters empty when `empty`),
    members at shuffled positions."""
    rng = np.random.default_rng(seed)
    out = np.empty((P, S), dtype=np.int32)
    for p in range(P):
        w = rng.uniform(lo, hi, C)
        if empty:
            w[rng.choice(C, size=max(1, C // 10), replace=False)] = 0.0
        sizes = np.floor(w / w.sum() * S).astype(np.int64)
        sizes[np.argmax(w)] += S - sizes.sum()
        lab = np.repeat(np.arange(C, dtype=np.int32), sizes)
        out[p] = lab[rng.permutation(S)]
    return out


# ------------------------------------------------------------------ layouts and probes


@pytest.mark.parametrize("P,S,C,seed", [(5, 3000, 40, 0), (3, 777, 300, 1), (80, 1100, 8, 2)])
def test_cluster_layouts_batched_bit_exact(bsa, P, S, C, seed):
    say(f"layouts P={P} S={S} C={C}")
    labels = head_labels(seed, P, S, C, 0.2, 3.0)
    labels[0] = 0  # one layout with a single non-empty cluster
    lay = bsa.cluster_layout(torch.from_numpy(labels).cuda(), C)
    assert lay.n_layouts == P
    perm, off, cnt = (t.cpu().numpy() for t in (lay.perm, lay.offsets, lay.counts))
    for p in range(P):
        rp, ro, rc = olay.cluster_layout(labels[p], C)
        assert np.array_equal(perm[p], rp) and np.array_equal(off[p], ro) and np.array_equal(cnt[p], rc), f"p={p}"


@pytest.mark.parametrize("S,C,M,lo,hi", [(3000, 40, 16, 0.5, 2.0), (3000, 40, 100, 0.5, 2.0), (400, 60, 300, 0.1, 3.0),
                                         (64, 64, 64, 1.0, 1.0)])
def test_select_probe_rows_layouts(bsa, S, C, M, lo, hi):
    """The device selection equals the host rule (bsa_select_probe_rows, the oracle's
    select_probe_rows) on every layout: a partial round (M below the non-empty clusters),
    full rounds with small and empty clusters, every member of every cluster taken."""
    say(f"probe selection S={S} C={C} M={M}")
    labels = head_labels(S + M, 4, S, C, lo, hi, empty=(lo < 1.0))
    lay = bsa.cluster_layout(torch.from_numpy(labels).cuda(), C)
    idx, w = (t.cpu().numpy() for t in bsa.select_probe_rows_layouts(lay, M))
    for p in range(4):
        ri, rw = orep.select_probe_rows(labels[p], C, M)
        assert np.array_equal(idx[p], ri), f"p={p}"
        np.testing.assert_allclose(w[p], rw, rtol=2e-6, atol=0)


# ------------------------------------------------------------------ attention


@pytest.mark.parametrize("dtype,D,Hq,Hkv,B,Hm,compensate", [("bf16", 128, 4, 2, 2, "kv", True),
                                                            ("bf16", 128, 4, 2, 1, "q", False),
                                                            ("f32", 64, 2, 2, 2, "q", True),
                                                            ("bf16", 64, 3, 1, 2, "kv", True)])
def test_attention_per_head_layouts(bsa, dtype, D, Hq, Hkv, B, Hm, compensate):
    """Compensated (and hard-drop) attention with its own query and key layouts per (batch,
    K/V head) against the oracle on each head's labels."""
    say(f"attention per-head layouts {dtype} D={D} Hq={Hq} Hkv={Hkv} B={B} Hm={Hm} comp={compensate}")
    S, C = 1300, 24
    wl = make_custom(70 + D + Hq, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype=dtype, mask="all")
    P = B * Hkv
    klab = head_labels(5 + D, P, S, C, 0.2, 3.0)
    qlab = head_labels(6 + D, P, S, C, 0.2, 3.0)
    H = Hkv if Hm == "kv" else Hq
    rng = np.random.default_rng(D + Hq)
    keep = (rng.random((B, H, C, C)) < 0.3).astype(np.uint8)
    keep[..., np.arange(C), np.arange(C)] = 1
    q, k, v = dev(wl.q, dtype), dev(wl.k, dtype), dev(wl.v, dtype)
    qlay = bsa.cluster_layout(torch.from_numpy(qlab.reshape(B, Hkv, S)).cuda(), C)
    klay = bsa.cluster_layout(torch.from_numpy(klab.reshape(B, Hkv, S)).cuda(), C)
    kv = bsa.kv_pack(k, v, klay)
    mask = bsa.mask_from_keep(torch.from_numpy(keep).cuda())
    out = host(bsa.block_sparse_attention(q, kv, qlay, mask, compensate, wl.scale))
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            kvh = hq // G
            p = b * Hkv + kvh
            hm = kvh if Hm == "kv" else hq
            ref, _ = oatt.compensated_attention(wl.q[b, hq], wl.k[b, kvh], wl.v[b, kvh], qlab[p], klab[p],
                                                keep[b, hm], wl.scale, compensate)
            check_output(out[b, hq], ref, dtype, f"per-head layouts b{b} h{hq}")


def test_shared_and_per_head_layouts_do_not_mix(bsa):
    wl = make_custom(3, B=1, Hq=2, Hkv=2, S=300, D=64, dtype="bf16", mask="all")
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    lab = head_labels(3, 2, 300, 8, 0.5, 2.0).reshape(1, 2, 300)
    per_head = bsa.cluster_layout(torch.from_numpy(lab).cuda(), 8)
    shared = bsa.cluster_layout(torch.from_numpy(lab[0, 0]).cuda(), 8)
    kv = bsa.kv_pack(k, v, per_head)
    mask = bsa.mask_from_keep(torch.ones(1, 2, 8, 8, dtype=torch.uint8).cuda())
    with pytest.raises(ValueError):
        bsa.block_sparse_attention(q, kv, shared, mask, True, wl.scale)
    # one mask row for every head cannot serve layouts that differ per head
    with pytest.raises(Exception):
        bsa.block_sparse_attention(q, kv, per_head, bsa.mask_from_keep(torch.ones(1, 1, 8, 8, dtype=torch.uint8).cuda()),
                                   True, wl.scale)


# ------------------------------------------------------------------ routing and repair


def test_routing_per_head_layouts(bsa):
    """The router's stages on per-head layouts: query-cluster probes, block errors and routes
    of every head against the oracle on that head's labels (routes outside near-tied rows)."""
    say("routing per-head layouts")
    B, Hq, Hkv, S, D, C = 1, 4, 2, 2000, 128, 20
    wl = make_custom(81, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", mask="all")
    P = B * Hkv
    klab = head_labels(82, P, S, C, 0.3, 2.5)
    qlab = head_labels(83, P, S, C, 0.3, 2.5)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    qlay = bsa.cluster_layout(torch.from_numpy(qlab.reshape(B, Hkv, S)).cuda(), C)
    klay = bsa.cluster_layout(torch.from_numpy(klab.reshape(B, Hkv, S)).cuda(), C)
    kv = bsa.kv_pack(k, v, klay)
    qbar = bsa.query_centroids(q, qlay)
    err = host(bsa.block_error(qbar, kv, wl.scale))
    budget = int(0.3 * S)
    keep = bsa.error_route(torch.from_numpy(err.astype(np.float32)).cuda(), klay, budget).keep.cpu().numpy()
    qbar_h = host(qbar)
    G = Hq // Hkv
    for h in range(Hq):
        p = h // G
        oq = ort.query_centroids(wl.q[:, h:h + 1], qlab[p], C)
        np.testing.assert_allclose(qbar_h[:, h:h + 1], oq, rtol=8e-3, atol=1e-6)  # rounded to bfloat16
        # block errors of the GPU's own probes (an input of the error pass)
        want = ort.block_compensation_error(qbar_h[:, h:h + 1], wl.k[:, p:p + 1], wl.v[:, p:p + 1], klab[p], C,
                                            wl.scale)
        bound = 1e-2 * want + 2e-3 * want.max(axis=-1, keepdims=True) + 1e-5 * np.abs(wl.v).max()
        assert np.all(np.abs(err[:, h:h + 1] - want) <= bound)
        n = np.bincount(klab[p], minlength=C)
        e32 = err[:, h:h + 1].astype(np.float32)
        want_keep = ort.error_aware_route(e32, n, budget)
        fragile = route_fragile_rows(e32, n, budget)[0, 0]
        same = np.all(keep[0, h] == want_keep[0, 0], axis=1)
        assert np.all(same | fragile), f"h{h}: {np.sum(~same & ~fragile)} routes differ outside near ties"


@pytest.mark.parametrize("M", [16, 40])
def test_probe_rows_and_fit_per_head_layouts(bsa, M):
    """Probe rows chosen per layout on the device, their dense and block-sparse rows from the
    per-head packed tiles, and the fit with each layout's weights, against the oracle."""
    say(f"probe rows and fit per-head layouts M={M}")
    B, Hq, Hkv, S, D, C = 2, 2, 1, 2500, 128, 30
    wl = make_custom(90 + M, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", mask="all")
    P = B * Hkv
    klab = head_labels(91, P, S, C, 0.3, 2.5)
    qlab = head_labels(92, P, S, C, 0.3, 2.5)
    rng = np.random.default_rng(M)
    keep = (rng.random((B, Hkv, C, C)) < 0.3).astype(np.uint8)
    keep[..., np.arange(C), np.arange(C)] = 1
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    qlay = bsa.cluster_layout(torch.from_numpy(qlab.reshape(B, Hkv, S)).cuda(), C)
    klay = bsa.cluster_layout(torch.from_numpy(klab.reshape(B, Hkv, S)).cuda(), C)
    kv = bsa.kv_pack(k, v, klay)
    mask = bsa.mask_from_keep(torch.from_numpy(keep).cuda())
    pidx, pw = bsa.select_probe_rows_layouts(qlay, M)
    od, os_ = bsa.probe_attention_packed(q, kv, pidx, wl.scale, q_labels=torch.from_numpy(qlab).cuda(), mask=mask,
                                         compensate=True)
    A, c = bsa.probe_fit(os_, od, pw, 0.1, 16)
    od, os_, A, c = host(od), host(os_), host(A), host(c)
    idx_h, w_h = pidx.cpu().numpy(), pw.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            p = b * Hkv + h // (Hq // Hkv)
            ri, rw = orep.select_probe_rows(qlab[p], C, M)
            assert np.array_equal(idx_h[p], ri)
            ref_d = oatt.dense_attention_rows(wl.q[b, h][ri], wl.k[b, 0], wl.v[b, 0], wl.scale)
            check_output(od[b, h], ref_d, "bf16", f"dense probe rows b{b} h{h}")
            ref_s, _ = oatt.compensated_attention(wl.q[b, h], wl.k[b, 0], wl.v[b, 0], qlab[p], klab[p], keep[b, 0],
                                                  wl.scale, True, rows=ri)
            check_output(os_[b, h], ref_s, "bf16", f"sparse probe rows b{b} h{h}")
            fit = orep.ridge_fit(os_[b, h], od[b, h], w_h[p], 0.1, 16)  # the fit of the GPU's probe rows
            scale = np.max(np.abs(fit["A"])) + 1e-30
            assert np.max(np.abs(A[b, h] - fit["A"])) <= 1e-4 * scale + 1e-6
            assert np.max(np.abs(c[b, h] - fit["c"])) <= 1e-4 * (np.max(np.abs(fit["c"])) + scale) + 1e-6


def test_path_partitioned(bsa):
    """SparsePR's call end to end (partitioned mode): response-coupled partitions, per-head
    layouts and packed tiles, error-aware routes with the probes' share reserved, per-layout
    probes, the fit and the corrected attention.  The partition itself is checked in
    test_gpu_partition; here the oracle takes the path's labels: the routes equal the oracle's
    on the path's probes outside near-tied rows, the probes follow the selection rule on the
    labels, and every output row matches the oracle's compensated attention with the fitted
    correction on the path's mask."""
    B, Hq, Hkv, S, D, C, M = 1, 2, 1, 2048, 128, 16, 16
    say("partitioned path")
    wl = make_custom(95, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", mask="all")
    cfg = bsa.PathConfig.from_workload(wl)
    cfg.mask_mode, cfg.C, cfg.route_density, cfg.probes, cfg.compensate = "partitioned", C, 0.3, M, True
    path = bsa.SparseAttentionPath(cfg)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    res = path(q, k, v)
    torch.cuda.synchronize()
    P = B * Hkv
    klab = res.extras["k_labels"].cpu().numpy().reshape(P, S)
    qlab = res.extras["q_labels"].cpu().numpy().reshape(P, S)
    assert klab.min() >= 0 and klab.max() < C and qlab.min() >= 0 and qlab.max() < C
    budget = res.extras["budget"]
    assert budget == int(round(0.3 * S)) - M
    keep = res.mask.keep.cpu().numpy()
    qbar = host(bsa.query_centroids(q, res.extras["q_layout"]))
    pidx, pw = res.extras["probe_idx"].cpu().numpy(), res.extras["probe_w"].cpu().numpy()
    out = host(res.out)
    G = Hq // Hkv
    for h in range(Hq):
        p = h // G
        n = np.bincount(klab[p], minlength=C)
        e = ort.block_compensation_error(qbar[:, h:h + 1], wl.k[:, p:p + 1], wl.v[:, p:p + 1], klab[p], C, wl.scale)
        e32 = e.astype(np.float32)
        same = np.all(keep[0, h] == ort.error_aware_route(e32, n, budget)[0, 0], axis=1)
        fragile = route_fragile_rows(e32, n, budget)[0, 0]
        assert np.all(same | fragile), f"h{h}: routes differ outside near ties"
        ri, rw = orep.select_probe_rows(qlab[p], C, M)
        assert np.array_equal(pidx[p], ri)
        np.testing.assert_allclose(pw[p], rw, rtol=2e-6)
        o_sparse, _ = oatt.compensated_attention(wl.q[0, h], wl.k[0, p], wl.v[0, p], qlab[p], klab[p], keep[0, h],
                                                 wl.scale, True)
        od = oatt.dense_attention_rows(wl.q[0, h][ri], wl.k[0, p], wl.v[0, p], wl.scale)
        fit = orep.ridge_fit(o_sparse[ri], od, rw, cfg.lam, cfg.rank)
        ref = orep.apply_correction(o_sparse, fit["A"], fit["c"])
        check_output(out[0, h], ref, "bf16", f"partitioned path h{h}")
