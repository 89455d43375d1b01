"""GPU parity, stage by stage: every kernel against the oracle on the same seeded inputs,
at sizes the oracle finishes in seconds that still span several tiles and ragged tails."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import centroids as ocen
from oracle import layout as olay
from oracle import repair as orep
from oracle import scoring as osco
from synthetic import bf16_bits, make_custom

from gpu_common import check_output, compare_masks, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


# ------------------------------------------------------------------ layout


@pytest.mark.parametrize("S,C,seed", [(1, 1, 0), (1000, 7, 1), (4096, 300, 2), (32760, 256, 3), (5000, 8192, 4)])
def test_cluster_layout_bit_exact(bsa, S, C, seed):
    say(f"layout S={S} C={C}")
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, C, size=S).astype(np.int32)
    if C > 2:
        labels[labels == 1] = 2  # an empty cluster
    lay = bsa.cluster_layout(torch.from_numpy(labels).cuda(), C)
    perm, off, cnt = olay.cluster_layout(labels, C)
    assert np.array_equal(lay.perm.cpu().numpy(), perm)
    assert np.array_equal(lay.offsets.cpu().numpy(), off)
    assert np.array_equal(lay.counts.cpu().numpy(), cnt)


# ------------------------------------------------------------------ centroids


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_centroids(bsa, dtype, D):
    say(f"centroids {dtype} D={D}")
    wl = make_custom(11, B=2, Hq=2, Hkv=2, S=1500, D=D, dtype=dtype)
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, wl.C)
    kbar, vbar = bsa.centroids(dev(wl.k, dtype), dev(wl.v, dtype), lay)
    for b in range(2):
        for h in range(2):
            kb, vb, n = ocen.centroids(wl.k[b, h], wl.v[b, h], wl.labels, wl.C)
            assert np.allclose(host(kbar[b, h]), kb, rtol=1e-5, atol=1e-6)
            assert np.allclose(host(vbar[b, h]), vb, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------------ K/V packing


def _align(x):
    return (x + 255) // 256 * 256


def decode_packed(buf: np.ndarray, B, Hkv, S, D, C, elem, nl=1):
    """Sections of the packed buffer as documented for bsa_kv_pack (test-side decoding):
    per-head format summary, tile flags, K and V tiles, then per layout the cluster tile
    offsets (returned [nl, C+1], or [C+1] for one layout) and the centroid log2 counts."""
    tok = -(-S // 64) + C
    ctiles = -(-C // 64)
    tph = tok + ctiles
    nt = B * Hkv * tph
    off_hmix = 0
    off_flags = off_hmix + _align(4 * B * Hkv)
    off_k = off_flags + _align(nt)
    off_v = off_k + _align(nt * 64 * D * elem)
    off_toff = off_v + _align(nt * 64 * D * elem)
    tile_off = buf[off_toff: off_toff + 4 * nl * (C + 1)].view(np.int32).reshape(nl, C + 1)
    if nl == 1:
        tile_off = tile_off[0]
    flags = buf[off_flags: off_flags + nt].reshape(B * Hkv, tph)
    kdt = np.uint16 if elem == 2 else np.float32
    kt = buf[off_k: off_k + nt * 64 * D * elem].view(kdt).reshape(B * Hkv, tph, 64, D)
    vt = buf[off_v: off_v + nt * 64 * D * elem].view(kdt).reshape(B * Hkv, tph, D, 64)
    # V^T positions hold the keys of each 16-key group in the order 0-3, 8-11, 4-7, 12-15
    pos = np.arange(64)
    key_at = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)
    vt_nat = np.empty_like(vt)
    vt_nat[..., key_at] = vt
    hmix = buf[off_hmix: off_hmix + 4 * B * Hkv].view(np.int32)
    return tile_off, flags, kt, vt_nat, tok, hmix


def _as_f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def scale_v_clusters(wl, scales):
    """Multiply V of whole clusters by powers of two (exact in bfloat16): {(b, kvh, c): 2^e}."""
    for (b, h, c), f in scales.items():
        wl.v[b, h][wl.labels == c] *= f
    return wl


MIXED = {(0, 0, 1): 2.0 ** 17, (0, 1, 2): 2.0 ** -14, (1, 0, 0): 2.0 ** 20}


def scale_v_alternate_tiles(wl, factor):
    """Multiply V of every second 64-key tile of each cluster (tiles 1, 3, ... in layout order)
    by a power of two, so that consecutive tiles of one cluster take different V^T formats."""
    perm, off, _ = olay.cluster_layout(wl.labels, wl.C)
    for c in range(wl.C):
        rows = perm[off[c]: off[c + 1]]
        for j in range(1, -(-rows.size // 64), 2):
            wl.v[:, :, rows[j * 64: (j + 1) * 64]] *= factor
    return wl


@pytest.mark.parametrize("dtype,D,sizes,mixed", [("bf16", 128, None, False), ("f32", 64, None, False),
                                                 ("bf16", 64, [0, 1, 63, 64, 65, 130, 7], False),
                                                 ("bf16", 128, None, True),
                                                 ("bf16", 128, [200, 150, 70, 64, 300, 129, 1], "tiles")])
def test_kv_pack(bsa, dtype, D, sizes, mixed):
    """Packed tiles hold every cluster's keys in layout order, zero-padded to 64, V^T as float16
    exactly when the tile's values fit (else bfloat16), and the centroid tiles; bit-exact.
    The "tiles" case alternates the format from tile to tile inside clusters of several tiles,
    so that each tile's format decision must not leak into its neighbour's."""
    say(f"kv pack {dtype} D={D} sizes={sizes} mixed={mixed}")
    if sizes is None:
        wl = make_custom(13, B=2, Hq=2, Hkv=2, S=1500, D=D, dtype=dtype)
        if mixed:
            scale_v_clusters(wl, MIXED)
    else:
        wl = make_custom(14, B=1 if mixed != "tiles" else 2, Hq=1, Hkv=1, S=sum(sizes), D=D, dtype=dtype,
                         cluster_sizes=sizes, shuffle_labels=True)
        if mixed == "tiles":
            scale_v_alternate_tiles(wl, 2.0 ** 17)
    B, Hkv, S, C = wl.B, wl.Hkv, wl.S, wl.C
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, C)
    kv = bsa.kv_pack(dev(wl.k, dtype), dev(wl.v, dtype), lay)
    elem = 2 if dtype == "bf16" else 4
    tile_off, flags, kt, vt, tok, hmix = decode_packed(kv.buffer.cpu().numpy(), B, Hkv, S, D, C, elem)
    perm, off, cnt = olay.cluster_layout(wl.labels, C)
    ntiles = -(-cnt // 64)
    assert np.array_equal(tile_off, np.concatenate([[0], np.cumsum(ntiles)]))
    kbar, vbar = host(kv.kbar), host(kv.vbar)
    for b in range(B):
        for h in range(Hkv):
            u = b * Hkv + h
            kb, vb, _ = ocen.centroids(wl.k[b, h], wl.v[b, h], wl.labels, C)
            # float32 sums: the rounding is relative to the terms' magnitude, not the mean's
            # (a cluster mixing tiles scaled by 2^17 with plain ones cancels to small means)
            ka, va, _ = ocen.centroids(np.abs(wl.k[b, h]), np.abs(wl.v[b, h]), wl.labels, C)
            assert np.all(np.abs(kbar[b, h] - kb) <= 1e-5 * ka + 1e-6)
            assert np.all(np.abs(vbar[b, h] - vb) <= 1e-5 * va + 1e-6)
            kbits = bf16_bits(wl.k[b, h]) if elem == 2 else wl.k[b, h].astype(np.float32)
            for c in range(C):
                rows = perm[off[c]: off[c + 1]]
                for j in range(ntiles[c]):
                    t = tile_off[c] + j
                    r = rows[j * 64: (j + 1) * 64]
                    n = r.size
                    assert np.array_equal(kt[u, t, :n], kbits[r]), (c, j)
                    assert not kt[u, t, n:].any()
                    vals = wl.v[b, h][r].astype(np.float64)  # [n, D], exact in the input type
                    if elem == 4:
                        assert flags[u, t] == 1
                        assert np.array_equal(vt[u, t, :, :n], vals.T.astype(np.float32))
                    else:
                        mx = np.max(np.abs(vals)) if n else 0.0
                        fits = mx < 65536.0 and mx >= 2.0 ** -8
                        assert flags[u, t] == int(fits), (c, j, mx)
                        want = _as_f16_bits(vals.T) if fits else bf16_bits(vals.T)
                        assert np.array_equal(vt[u, t, :, :n], want), (c, j)
                    assert not vt[u, t, :, n:].any()
            # centroid tiles: K-bar rounded to the input type, V-bar^T like value tiles
            for j in range(-(-C // 64)):
                t = tok + j
                cs = slice(j * 64, min(C, (j + 1) * 64))
                n = cs.stop - cs.start
                want_k = bf16_bits(kbar[b, h][cs]) if elem == 2 else kbar[b, h][cs].astype(np.float32)
                assert np.array_equal(kt[u, t, :n], want_k)
                vv = vbar[b, h][cs]
                if elem == 2:
                    mx = np.max(np.abs(vv))
                    fits = mx <= 65504.0 and mx >= 2.0 ** -8
                    assert flags[u, t] == int(fits)
                    want_v = _as_f16_bits(vv.T) if fits else bf16_bits(vv.T)
                else:
                    want_v = vv.T.astype(np.float32)
                assert np.array_equal(vt[u, t, :, :n], want_v)
            # per-head summary: nonzero exactly when some token or centroid V^T tile is bfloat16
            used = [tile_off[c] + j for c in range(C) for j in range(ntiles[c])] + \
                [tok + j for j in range(-(-C // 64))]
            assert (hmix[u] != 0) == bool(np.any(flags[u, used] == 0)), (b, h)


# ------------------------------------------------------------------ top-p


# Rows of at most 256 clusters take the one-wave-per-row kernel (four rows per workgroup; 41
# query blocks leave a part-filled last workgroup), wider rows the workgroup-per-row kernel.
@pytest.mark.parametrize("Ck,seed,Cq", [(1, 0, 40), (16, 1, 40), (32, 2, 40), (200, 5, 41), (256, 3, 40),
                                        (257, 6, 41), (1000, 4, 40)])
def test_top_p(bsa, Ck, seed, Cq):
    say(f"top-p Ck={Ck} Cq={Cq}")
    rng = np.random.default_rng(seed)
    B, Hs = 2, 3
    scores = rng.dirichlet(np.full(Ck, 0.3), size=(B, Hs, Cq)).astype(np.float32)
    scores[0, 0, 0] = 1.0 / Ck  # an all-equal row: ties by lower index
    taus = np.array([0.85, 0.9, 0.95], dtype=np.float32)
    mask = bsa.top_p_block_mask(torch.from_numpy(scores).cuda(), taus)
    keep, cnt, idx = mask.keep.cpu().numpy(), mask.kv_count.cpu().numpy(), mask.kv_idx.cpu().numpy()
    for b in range(B):
        for h in range(Hs):
            # Both sides sort the same float32 scores, so only the prefix sums round apart.  The
            # 1000-cluster Dirichlet rows put many tiny scores at the cut: up to 15% of their
            # rows decide a block within 1e-5 of tau.
            compare_masks(keep[b, h], cnt[b, h], idx[b, h], scores[b, h].astype(np.float64), float(taus[h]),
                          f"top-p b{b} h{h}", eps_tie=0.0, max_fragile=0.15 if Ck > 256 else 0.10)
    assert cnt.min() >= 1


def test_mask_lists(bsa):
    say("mask lists")
    rng = np.random.default_rng(5)
    keep = (rng.uniform(size=(2, 3, 17, 300)) < 0.3).astype(np.uint8)
    m = bsa.mask_from_keep(torch.from_numpy(keep).cuda())
    cnt, idx = m.kv_count.cpu().numpy(), m.kv_idx.cpu().numpy()
    for r, row in enumerate(keep.reshape(-1, 300)):
        want = np.nonzero(row)[0]
        assert cnt.reshape(-1)[r] == want.size
        assert np.array_equal(idx.reshape(-1, 300)[r, : want.size], want)


# ------------------------------------------------------------------ scores


@pytest.mark.parametrize(
    "S,D,block,stride,dtype,Hq,Hkv,shuffle",
    [
        (1000, 128, 128, 16, "bf16", 2, 2, True),    # ragged tail, padded keys, gathered order
        (4096, 128, 128, 16, "bf16", 2, 1, False),   # two 128-row tiles of strided rows
        (2048, 64, 64, 8, "f32", 2, 2, True),        # R = 8, D = 64, float32
        (777, 128, 64, 16, "bf16", 2, 2, False),     # R = 4
        (900, 64, 32, 16, "bf16", 1, 1, True),       # R = 2
        (3000, 128, 256, 16, "bf16", 1, 1, False),   # R = 16
        (10000, 128, 128, 16, "bf16", 2, 1, True),   # three 256-row tiles of strided rows, ragged
        (9000, 64, 64, 4, "f32", 1, 1, True),        # stride 4: nine tiles, float32
    ],
)
def test_antidiagonal_scores_and_mask(bsa, S, D, block, stride, dtype, Hq, Hkv, shuffle):
    say(f"scores S={S} D={D} block={block} stride={stride} {dtype}")
    wl = make_custom(21 + S, B=1, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype=dtype, block=block, mask="scored", noise=0.8)
    labels = wl.labels.copy()
    perm_np = None
    if shuffle:
        # Cluster-major order of shuffled positions: label = rank // block of a random order.
        order = np.random.default_rng(S).permutation(S)
        labels = np.empty(S, dtype=np.int32)
        labels[order] = np.arange(S) // block
    C = -(-S // block)
    lay = bsa.cluster_layout(torch.from_numpy(labels.astype(np.int32)).cuda(), C)
    perm_np = olay.cluster_layout(labels, C)[0]
    q, k = dev(wl.q, dtype), dev(wl.k, dtype)
    pool = Hq != Hkv
    scores = bsa.antidiagonal_block_scores(q, k, lay, block, stride, 1 / math.sqrt(D), pool_gqa=pool)
    got = host(scores)
    taus = np.array([0.9] * scores.shape[1], dtype=np.float32)
    mask = bsa.top_p_block_mask(scores, taus)
    keep, cnt, idx = mask.keep.cpu().numpy(), mask.kv_count.cpu().numpy(), mask.kv_idx.cpu().numpy()
    for hs in range(scores.shape[1]):
        if pool:
            g = Hq // Hkv
            ref = np.mean([osco.antidiagonal_block_scores(wl.q[0, h], wl.k[0, hs], perm_np, block, stride,
                                                          1 / math.sqrt(D)) for h in range(hs * g, (hs + 1) * g)], 0)
        else:
            ref = osco.antidiagonal_block_scores(wl.q[0, hs], wl.k[0, hs * Hkv // Hq], perm_np, block, stride,
                                                 1 / math.sqrt(D))
        assert np.allclose(got[0, hs], ref, rtol=1e-4, atol=1e-6), np.max(np.abs(got[0, hs] - ref))
        compare_masks(keep[0, hs], cnt[0, hs], idx[0, hs], ref, 0.9, f"scores head {hs}")


# ------------------------------------------------------------------ attention


def run_attention(bsa, wl, keep_np, compensate, lse=False):
    dtype = wl.dtype
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, wl.C)
    q, k, v = dev(wl.q, dtype), dev(wl.k, dtype), dev(wl.v, dtype)
    mask = bsa.mask_from_keep(torch.from_numpy(np.ascontiguousarray(keep_np)).cuda())
    return bsa.centroid_compensated_attention(q, k, v, lay, lay, mask, compensate, wl.scale, return_lse=lse)


def oracle_attention(wl, keep_np, compensate, b, hq):
    Hm = keep_np.shape[1]
    hm = 0 if Hm == 1 else (hq if Hm == wl.Hq else hq // (wl.Hq // wl.Hkv))
    kvh = hq // (wl.Hq // wl.Hkv)
    return oatt.compensated_attention(wl.q[b, hq], wl.k[b, kvh], wl.v[b, kvh], wl.labels, wl.labels,
                                      keep_np[b, hm], wl.scale, compensate)


@pytest.mark.parametrize(
    "name,kw,compensate",
    [
        ("ragged_bf16_d128", dict(S=1500, D=128, dtype="bf16"), True),
        ("ragged_bf16_d128_harddrop", dict(S=1500, D=128, dtype="bf16"), False),
        ("ragged_f32_d64", dict(S=900, D=64, dtype="f32"), True),
        ("ragged_f32_d128", dict(S=700, D=128, dtype="f32"), True),
        ("ragged_bf16_d64", dict(S=1100, D=64, dtype="bf16"), True),
        ("gqa_bf16", dict(S=1200, D=128, dtype="bf16", Hq=4, Hkv=2, B=2), True),
        ("big_clusters", dict(S=1000, D=128, dtype="bf16", cluster_sizes=[300, 5, 129, 64, 1, 257, 244]), True),
        ("all_kept", dict(S=1000, D=128, dtype="bf16", mask="all"), True),
        ("nothing_kept_compensated", dict(S=1000, D=128, dtype="bf16", mask="none"), True),
        ("student_t_values", dict(S=1300, D=128, dtype="bf16", v_kind="t3"), True),
        # heads whose V holds tiles outside float16's range next to all-float16 heads
        ("mixed_v_formats", dict(S=1500, D=128, dtype="bf16", Hq=2, Hkv=2, B=2), True),
    ],
)
def test_sparse_attention(bsa, name, kw, compensate):
    say(f"attention {name}")
    wl = make_custom(100 + len(name), **kw)
    if name == "mixed_v_formats":
        scale_v_clusters(wl, MIXED)
    out, lse = run_attention(bsa, wl, wl.mask, compensate, lse=True)
    got = host(out)
    got_lse = lse.cpu().numpy()
    for b in range(wl.B):
        for hq in range(wl.Hq):
            ref, ref_lse = oracle_attention(wl, wl.mask, compensate, b, hq)
            check_output(got[b, hq], ref, wl.dtype, f"{name} b{b} h{hq}")
            fin = np.isfinite(ref_lse)
            assert np.array_equal(np.isfinite(got_lse[b, hq]), fin)
            # bf16: centroids enter the MFMA rounded to bf16, which moves centroid logits by
            # up to ~1e-3; float32 keeps them exact to rounding.
            lse_tol = 1e-4 if wl.dtype == "f32" else 1e-2
            assert np.max(np.abs(got_lse[b, hq][fin] - ref_lse[fin])) < lse_tol


@pytest.mark.parametrize("grid,tile,window,compensate", [((4, 16, 24), (2, 8, 8), (1, 2, 3), True),
                                                         ((5, 18, 20), (2, 8, 8), (3, 1, 3), True),
                                                         ((5, 18, 20), (2, 8, 8), (1, 3, 1), False)])
def test_attention_sliding_tile_mask(bsa, grid, tile, window, compensate):
    """Static sliding-tile masks ([SBC] "Recipe: STA with both repairs"): tile labels as the
    clusters (edge tiles partial on the second grid), the tile-level mask from the host
    helper, compensated and hard-drop attention against the oracle with the oracle's mask."""
    from oracle import layout as olay
    from oracle import static_masks as osm
    T, H, W = grid
    say(f"attention sliding tile grid={grid} tile={tile} window={window} compensate={compensate}")
    wl = make_custom(90 + sum(grid), B=1, Hq=2, Hkv=2, S=T * H * W, D=128, dtype="bf16", mask="all")
    wl.labels = olay.tile_labels(T, H, W, tile)
    wl.C = int(wl.labels.max()) + 1
    nt, nh, nw = -(-T // tile[0]), -(-H // tile[1]), -(-W // tile[2])
    keep_tile = bsa.sliding_tile_block_mask(nt, nh, nw, (1, 1, 1), window)
    assert np.array_equal(keep_tile, osm.sliding_tile_block_mask(nt, nh, nw, (1, 1, 1), window))
    keep = np.broadcast_to(keep_tile, (1, wl.Hkv) + keep_tile.shape).copy()
    out = host(run_attention(bsa, wl, keep, compensate))
    oracle_keep = np.broadcast_to(osm.sliding_tile_block_mask(nt, nh, nw, (1, 1, 1), window),
                                  (1, wl.Hkv, wl.C, wl.C))
    for hq in range(wl.Hq):
        ref, _ = oracle_attention(wl, oracle_keep, compensate, 0, hq)
        check_output(out[0, hq], ref, "bf16", f"sliding tile h{hq}")


def test_hard_drop_empty_rows_are_zero(bsa):
    say("attention empty rows")
    wl = make_custom(7, S=600, D=128, dtype="bf16", mask="random", p_keep=0.2)
    keep = wl.mask.copy()
    keep[0, 0, 0] = 0  # cluster 0 keeps nothing
    out, lse = run_attention(bsa, wl, keep, compensate=False, lse=True)
    rows = wl.labels == 0
    assert np.all(host(out)[0, 0][rows] == 0)
    assert np.all(np.isneginf(lse.cpu().numpy()[0, 0][rows]))
    ref, _ = oracle_attention(wl, keep, False, 0, 0)
    check_output(host(out)[0, 0], ref, "bf16", "empty rows")


def test_identical_keys_compensation_equals_dense(bsa):
    say("attention identical keys")
    wl = make_custom(8, S=1024, D=128, dtype="f32", noise=0.0, mask="random", p_keep=0.2)
    # keys identical within each cluster: compensation is exact
    for c in range(wl.C):
        rows = wl.labels == c
        wl.k[0, 0][rows] = wl.k[0, 0][rows][0]
    out = host(run_attention(bsa, wl, wl.mask, compensate=True))
    dense = oatt.dense_attention_rows(wl.q[0, 0], wl.k[0, 0], wl.v[0, 0], wl.scale)
    check_output(out[0, 0], dense, "f32", "identical keys vs dense")


# ------------------------------------------------------------------ probes, fit, apply


@pytest.mark.parametrize("dtype,D,M,compensate,Hkv", [("bf16", 128, 64, True, 1), ("f32", 64, 20, True, 2),
                                                      ("bf16", 128, 130, False, 1), ("bf16", 64, 33, True, 2)])
def test_probe_attention(bsa, dtype, D, M, compensate, Hkv):
    say(f"probe rows {dtype} D={D} M={M} compensate={compensate}")
    wl = make_custom(31 + M, B=1, Hq=2, Hkv=Hkv, S=5000, D=D, dtype=dtype, p_keep=0.25)
    idx = np.random.default_rng(0).choice(wl.S, size=M, replace=False).astype(np.int32)
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, wl.C)
    q, k, v = dev(wl.q, dtype), dev(wl.k, dtype), dev(wl.v, dtype)
    mask = bsa.mask_from_keep(torch.from_numpy(wl.mask).cuda())
    kbar = vbar = None
    if compensate:
        kbar, vbar = bsa.centroids(k, v, lay)
    od, os_ = bsa.probe_attention(q, k, v, torch.from_numpy(idx).cuda(), wl.scale, lab, lab, lay, mask, kbar, vbar)
    od, os_ = host(od), host(os_)
    for h in range(2):
        kvh = h // (2 // Hkv)
        ref = oatt.dense_attention_rows(wl.q[0, h][idx], wl.k[0, kvh], wl.v[0, kvh], wl.scale)
        check_output(od[0, h], ref, dtype, f"dense probe rows h{h}")
        ref_s, _ = oatt.compensated_attention(wl.q[0, h], wl.k[0, kvh], wl.v[0, kvh], wl.labels, wl.labels,
                                              wl.mask[0, kvh if Hkv > 1 else 0], wl.scale, compensate, rows=idx)
        check_output(os_[0, h], ref_s, dtype, f"sparse probe rows h{h}")


@pytest.mark.parametrize("D,M,Hkv,sizes,mixed", [(128, 64, 1, None, False), (64, 33, 2, None, False),
                                                   (128, 130, 2, None, True),
                                                   (128, 64, 1, [0, 1, 63, 64, 65, 130, 7, 1000, 3000], False)])
def test_probe_attention_packed(bsa, D, M, Hkv, sizes, mixed):
    """Probe rows from the packed tiles against the oracle: the dense rows, and the same probes
    under the block-sparse rule (compensated and hard drop) from the same pass; ragged and empty
    clusters (the last tile of a cluster is partial), several row tiles (M = 130: 260 rows),
    and heads whose V^T tiles are partly bfloat16 (values outside the float16 range)."""
    say(f"probe rows from packed tiles D={D} M={M} Hkv={Hkv} sizes={sizes} mixed={mixed}")
    if sizes is None:
        wl = make_custom(41 + M, B=1, Hq=2, Hkv=Hkv, S=5000, D=D, dtype="bf16")
        if mixed:
            scale_v_clusters(wl, {key: f for key, f in MIXED.items() if key[0] < wl.B and key[1] < wl.Hkv})
    else:
        wl = make_custom(42, B=1, Hq=2, Hkv=Hkv, S=sum(sizes), D=D, dtype="bf16", cluster_sizes=sizes,
                         shuffle_labels=True)
    idx = np.random.default_rng(1).choice(wl.S, size=M, replace=False).astype(np.int32)
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    kv = bsa.kv_pack(k, v, lay)
    pidx = torch.from_numpy(idx).cuda()
    od = host(bsa.probe_attention_packed(q, kv, pidx, wl.scale))
    for h in range(2):
        kvh = h // (2 // Hkv)
        ref = oatt.dense_attention_rows(wl.q[0, h][idx], wl.k[0, kvh], wl.v[0, kvh], wl.scale)
        check_output(od[0, h], ref, "bf16", f"dense probe rows (packed) h{h}")
    mask = bsa.mask_from_keep(torch.from_numpy(wl.mask).cuda())  # one mask per K/V head
    lab = torch.from_numpy(wl.labels).cuda()
    for comp in (True, False):
        od2, os_ = bsa.probe_attention_packed(q, kv, pidx, wl.scale, q_labels=lab, mask=mask, compensate=comp)
        od2, os_ = host(od2), host(os_)
        for h in range(2):
            kvh = h // (2 // Hkv)
            ref = oatt.dense_attention_rows(wl.q[0, h][idx], wl.k[0, kvh], wl.v[0, kvh], wl.scale)
            check_output(od2[0, h], ref, "bf16", f"dense probe rows beside sparse ones h{h}")
            ref_s, _ = oatt.compensated_attention(wl.q[0, h], wl.k[0, kvh], wl.v[0, kvh], wl.labels, wl.labels,
                                                  wl.mask[0, kvh], wl.scale, comp, rows=idx)
            check_output(os_[0, h], ref_s, "bf16", f"sparse probe rows (packed, comp={comp}) h{h}")


def fit_inputs(M, D, H=3, seed=0):
    rng = np.random.default_rng(seed)
    xs = rng.standard_normal((1, H, M, D)) * rng.uniform(0.3, 2.0, size=D)
    mix = rng.standard_normal((D, D)) * 0.05
    xd = xs + xs @ mix + 0.05 * rng.standard_normal((1, H, M, D)) + 0.1
    _, w = orep.select_probe_rows(np.arange(50 * 12) // 50, 12, M)
    return xs.astype(np.float32), xd.astype(np.float32), w.astype(np.float32)


# M <= 64: the dual M x M form; M > 64: the primal D x D form (probe rows streamed).
@pytest.mark.parametrize("D,M,rank", [(128, 64, 16), (64, 16, 4), (128, 2, 16), (128, 33, 16), (64, 64, 16),
                                      (128, 65, 16), (64, 96, 16), (128, 300, 12), (64, 520, 16)])
def test_probe_fit(bsa, D, M, rank):
    say(f"probe fit D={D} M={M} r={rank}")
    xs, xd, w = fit_inputs(M, D, seed=M + D)
    A, c = bsa.probe_fit(torch.from_numpy(xs).cuda(), torch.from_numpy(xd).cuda(), torch.from_numpy(w).cuda(),
                         0.1, rank)
    A_h, c_h = host(A), host(c)
    for h in range(xs.shape[1]):
        fit = orep.ridge_fit(xs[0, h], xd[0, h], w, 0.1, rank)
        scale = np.max(np.abs(fit["A"])) + 1e-30
        assert np.max(np.abs(A_h[0, h] - fit["A"])) <= 1e-4 * scale + 1e-6, np.max(np.abs(A_h[0, h] - fit["A"]))
        assert np.max(np.abs(c_h[0, h] - fit["c"])) <= 1e-4 * (np.max(np.abs(fit["c"])) + scale) + 1e-6


@pytest.mark.parametrize("D,M", [(64, 100), (128, 40), (128, 200)])
def test_probe_fit_low_rank(bsa, D, M):
    """A residual of rank 3 (plus a constant): three directions pass the 1e-12 eigenvalue
    threshold, so the rank-16 fit keeps 3; one feature has no spread (sigma taken as 1)."""
    say(f"probe fit low-rank residual D={D} M={M}")
    rng = np.random.default_rng(D + M)
    xs = rng.standard_normal((1, 2, M, D)) * rng.uniform(0.3, 2.0, size=D)
    xs[..., 5] = 0.75
    U = rng.standard_normal((D, 3))
    V = rng.standard_normal((3, D)) * 0.1
    xd = xs + (xs @ U) @ V + 0.2
    xs, xd = xs.astype(np.float32), xd.astype(np.float32)
    w = rng.uniform(0.5, 2.0, size=M).astype(np.float32)
    A, c = bsa.probe_fit(torch.from_numpy(xs).cuda(), torch.from_numpy(xd).cuda(), torch.from_numpy(w).cuda(), 0.1, 16)
    A_h, c_h = host(A), host(c)
    for h in range(2):
        fit = orep.ridge_fit(xs[0, h], xd[0, h], w, 0.1, 16)
        assert fit["r_eff"] == 3
        scale = np.max(np.abs(fit["A"])) + 1e-30
        assert np.max(np.abs(A_h[0, h] - fit["A"])) <= 1e-4 * scale + 1e-6, np.max(np.abs(A_h[0, h] - fit["A"]))
        assert np.max(np.abs(c_h[0, h] - fit["c"])) <= 1e-4 * (np.max(np.abs(fit["c"])) + scale) + 1e-6


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_probe_apply(bsa, dtype, D):
    say(f"probe apply {dtype} D={D}")
    rng = np.random.default_rng(D)
    B, H, S = 1, 2, 700
    o = rng.standard_normal((B, H, S, D)).astype(np.float32)
    A = (rng.standard_normal((B, H, D, D)) * 0.3).astype(np.float32)
    c = rng.standard_normal((B, H, D)).astype(np.float32)
    o_t = dev(o, dtype)
    before = host(o_t)
    bsa.probe_apply(o_t, torch.from_numpy(A).cuda(), torch.from_numpy(c).cuda())
    after = host(o_t)
    for h in range(H):
        check_output(after[0, h], orep.apply_correction(before[0, h], A[0, h], c[0, h]), dtype, f"apply h{h}")


def test_gather_rows_bit_exact(bsa):
    say("gather rows")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 300, 64)).astype(np.float32)
    idx = np.array([0, 299, 17, 150, 17], dtype=np.int32)
    got = bsa.gather_rows(torch.from_numpy(x).cuda(), torch.from_numpy(idx).cuda()).cpu().numpy()
    assert np.array_equal(got, x[:, :, idx])


@pytest.mark.parametrize("dtype,D,compensate", [("bf16", 128, True), ("f32", 64, True), ("bf16", 64, False)])
def test_attention_with_correction_epilogue(bsa, dtype, D, compensate):
    """The attention's repair epilogue: every row o leaves as o + o A + c, which equals the
    oracle's correction of its exact attention output (one rounding, at the end)."""
    say(f"attention epilogue {dtype} D={D}")
    wl = make_custom(77, B=1, Hq=2, Hkv=1, S=1200, D=D, dtype=dtype)
    rng = np.random.default_rng(3)
    A = (rng.standard_normal((1, 2, D, D)) * 0.5).astype(np.float32)
    c = (rng.standard_normal((1, 2, D)) * 0.1).astype(np.float32)
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, wl.C)
    q, k, v = dev(wl.q, dtype), dev(wl.k, dtype), dev(wl.v, dtype)
    mask = bsa.mask_from_keep(torch.from_numpy(wl.mask).cuda())
    out = host(bsa.centroid_compensated_attention(q, k, v, lay, lay, mask, compensate, wl.scale,
                                                  A=torch.from_numpy(A).cuda(), c=torch.from_numpy(c).cuda()))
    for h in range(2):
        ref, _ = oracle_attention(wl, wl.mask, compensate, 0, h)
        check_output(out[0, h], orep.apply_correction(ref, A[0, h], c[0, h]), dtype, f"epilogue h{h}")


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 2, 1), ("bf16", 64, 2, 2), ("f32", 128, 1, 1)])
def test_attention_caller_centroids(bsa, dtype, D, Hq, Hkv):
    """Centroid columns given by the caller (kv_pack_centroids): arbitrary centroids and counts,
    a count of 0 included (its column vanishes), against the oracle's extended-key softmax with
    the same columns; with the repair epilogue on top for bfloat16."""
    say(f"caller centroids {dtype} D={D} Hq={Hq} Hkv={Hkv}")
    wl = make_custom(91, B=1, Hq=Hq, Hkv=Hkv, S=1400, D=D, dtype=dtype)
    rng = np.random.default_rng(5)
    kb = (rng.standard_normal((1, Hkv, wl.C, D)) * 0.8).astype(np.float32)
    vb = rng.standard_normal((1, Hkv, wl.C, D)).astype(np.float32)
    n = rng.integers(0, 300, wl.C).astype(np.int32)
    n[1] = 0
    lab = torch.from_numpy(wl.labels).cuda()
    lay = bsa.cluster_layout(lab, wl.C)
    q, k, v = dev(wl.q, dtype), dev(wl.k, dtype), dev(wl.v, dtype)
    mask = bsa.mask_from_keep(torch.from_numpy(wl.mask).cuda())
    corr = dtype == "bf16"
    A = (rng.standard_normal((1, Hq, D, D)) * 0.3).astype(np.float32) if corr else None
    c = (rng.standard_normal((1, Hq, D)) * 0.1).astype(np.float32) if corr else None
    out = host(bsa.centroid_compensated_attention(
        q, k, v, lay, lay, mask, True, wl.scale, kbar=torch.from_numpy(kb).cuda(), vbar=torch.from_numpy(vb).cuda(),
        counts=torch.from_numpy(n).cuda(), A=torch.from_numpy(A).cuda() if corr else None,
        c=torch.from_numpy(c).cuda() if corr else None))
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        ref, _ = oatt.compensated_attention(wl.q[0, h], wl.k[0, kvh], wl.v[0, kvh], wl.labels, wl.labels,
                                            wl.mask[0, kvh], wl.scale, True, kbar=kb[0, kvh], vbar=vb[0, kvh],
                                            counts=n)
        if corr:
            ref = orep.apply_correction(ref, A[0, h], c[0, h])
        check_output(out[0, h], ref, dtype, f"caller centroids h{h}")
