"""C-ABI checks that need no GPU: the library loads, exports every declared entry point,
its host helpers agree with the oracle, and invalid calls are rejected on the host before
any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_antidiagonal_amd import _lib

    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for must in ("bsa_cluster_layout", "bsa_centroids", "bsa_antidiag_scores", "bsa_top_p_mask",
                 "bsa_sparse_attention", "bsa_probe_attention", "bsa_probe_fit", "bsa_probe_apply",
                 "bsa_select_probe_rows", "bsa_tile_labels"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    from block_sparse_attention_antidiagonal_amd import _lib

    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_status_strings_and_version(lib):
    assert lib.bsa_abi_version() == 4
    assert lib.bsa_status_string(0) == b"ok"
    assert b"workspace" in lib.bsa_status_string(5)


def test_probe_selection_matches_oracle():
    from block_sparse_attention_antidiagonal_amd import api
    from oracle import repair

    rng = np.random.default_rng(0)
    for C, S, M in ((9, 400, 64), (256, 32760, 64), (3, 10, 5), (40, 500, 40), (7, 30, 30)):
        labels = rng.integers(0, C, size=S).astype(np.int32)
        idx, w = api.select_probe_rows(labels, C, M)
        ridx, rw = repair.select_probe_rows(labels, C, M)
        assert np.array_equal(idx, ridx)
        assert np.allclose(w, rw, rtol=1e-6, atol=0)


def test_probe_selection_on_video_labels_matches_oracle():
    from block_sparse_attention_antidiagonal_amd import api
    from oracle import repair
    from synthetic import grid_tile_labels

    labels = grid_tile_labels(21, 30, 52, (2, 8, 8), 128)
    idx, w = api.select_probe_rows(labels, 256, 64)
    ridx, rw = repair.select_probe_rows(labels, 256, 64)
    assert np.array_equal(idx, ridx) and np.allclose(w, rw, rtol=1e-6)


def test_tile_labels_match_oracle_and_inputs():
    from block_sparse_attention_antidiagonal_amd import api
    from oracle import layout
    from synthetic import grid_tile_labels

    for T, H, W, tile, chunk in ((2, 3, 4, (1, 2, 2), 0), (2, 3, 4, (1, 2, 2), 3), (5, 7, 9, (2, 3, 4), 11),
                                 (21, 30, 52, (2, 8, 8), 128)):
        got = api.tile_labels(T, H, W, tile, chunk)
        assert np.array_equal(got, layout.tile_labels(T, H, W, tile, chunk))
        assert np.array_equal(got, grid_tile_labels(T, H, W, tile, chunk))


def test_video_labels_are_256_clusters_of_128():
    from synthetic import grid_tile_labels

    lab = grid_tile_labels(21, 30, 52, (2, 8, 8), 128)
    counts = np.bincount(lab)
    assert counts.size == 256 and np.all(counts[:-1] == 128) and counts[-1] == 120


def test_host_validation_rejects_before_launch(lib):
    dummy = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    size = ctypes.c_size_t(0)
    # unknown dtype
    assert lib.bsa_centroids(1, 1, 8, 128, 7, dummy, dummy, dummy, dummy, 1, dummy, dummy, None) == 3
    # sparse attention: (B, Hq, Hkv, S, D, dtype, Q, scale, q_perm, q_offsets, Cq, k_offsets, Ck, n_layouts,
    # keep, kv_count, kv_idx, Hm, packed, packed_bytes, compensate, A, c, out_dtype, O, lse, ws, ws_bytes,
    # stream)
    f = ctypes.c_float(0.1)
    big = 1 << 40
    # unsupported head dim
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 96, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, None, None, 1, dummy, None, dummy, big, None) == 4
    # Hq not a multiple of Hkv
    assert lib.bsa_sparse_attention(1, 3, 2, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, None, None, 1, dummy, None, dummy, big, None) == 2
    # output type must be the input type or float32; no packed buffer; packed buffer too small
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 0, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, None, None, 1, dummy, None, dummy, big, None) == 3
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, None, None, 9, dummy, None, dummy, big, None) == 3
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, None, big, 1, None, None, 1, dummy, None, dummy, big, None) == 1
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, 1024, 1, None, None, 1, dummy, None, dummy, big, None) == 5
    # attention workspace too small
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, None, None, 1, dummy, None, dummy, 16, None) == 5
    # the allocation-free call: a problem needing more than the static scratch (the video shape
    # with 200 heads needs about 165 MiB of tile lists)
    assert lib.bsa_sparse_attention_noalloc(1, 200, 200, 32760, 128, 1, dummy, f, dummy, dummy, 256, dummy, 256, 1, dummy, dummy, dummy, 200, dummy, big, 1, None, None, 1, dummy, None, None) == 5
    # repair epilogue: A without c; float32 rows with the epilogue
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, dummy, None, 1, dummy, None, dummy, big, None) == 1
    assert lib.bsa_sparse_attention(1, 1, 1, 8, 128, 1, dummy, f, dummy, dummy, 1, dummy, 1, 1, dummy, dummy, dummy, 1, dummy, big, 1, dummy, dummy, 0, dummy, None, dummy, big, None) == 4
    # caller centroids: counts are required; buffer too small
    assert lib.bsa_kv_pack_centroids(1, 1, 8, 128, 1, dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, None, dummy, big, None) == 1
    assert lib.bsa_kv_pack_centroids(1, 1, 8, 128, 1, dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, dummy, dummy, 64, None) == 5
    # K/V packing: centroid outputs are required; buffer too small; unsupported head dim
    assert lib.bsa_kv_pack(1, 1, 8, 128, 1, dummy, dummy, dummy, dummy, 1, 1, None, None, dummy, big, None) == 1
    assert lib.bsa_kv_pack(1, 1, 8, 128, 1, dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, dummy, 64, None) == 5
    assert lib.bsa_kv_pack(1, 1, 8, 80, 1, dummy, dummy, dummy, dummy, 1, 1, dummy, dummy, dummy, big, None) == 4
    # probe rows: sparse rows need the mask; too many key clusters
    assert lib.bsa_probe_attention(1, 1, 1, 8, 128, 1, dummy, dummy, dummy, ctypes.c_float(0.1), dummy, 4, None,
                                   None, None, 1, 1, 1, None, None, None, dummy, dummy, dummy, 1 << 30, None) == 1
    assert lib.bsa_probe_attention(1, 1, 1, 8, 128, 1, dummy, dummy, dummy, ctypes.c_float(0.1), dummy, 4, dummy,
                                   dummy, dummy, 1, 1, 4096, dummy, None, None, dummy, dummy, dummy, 1 << 30,
                                   None) == 4
    # null output; correction: unsupported head dim, null input
    assert lib.bsa_probe_apply(1, 1, 8, 128, 1, None, dummy, dummy, None) == 1
    assert lib.bsa_correct(1, 1, 8, 96, 1, dummy, dummy, dummy, dummy, None) == 4
    assert lib.bsa_correct(1, 1, 8, 128, 1, None, dummy, dummy, dummy, None) == 1
    assert lib.bsa_gather_rows(1, 8, 128, dummy, None, 4, dummy, None) == 1
    # block not a multiple of stride
    assert lib.bsa_antidiag_scores_workspace_size(1, 1, 1, 1024, 128, 100, 16, ctypes.byref(size)) == 1
    # workspace too small
    assert lib.bsa_cluster_layout(1, dummy, 100, 4, dummy, dummy, dummy, dummy, 0, None) == 5
    # too many probes for the fit; bad lambda
    assert lib.bsa_probe_fit(1, 1, 1, 128, dummy, dummy, dummy, 65537, 1, ctypes.c_float(0.1), 16, dummy, dummy, None) == 4
    assert lib.bsa_probe_fit(1, 1, 1, 128, dummy, dummy, dummy, 64, 1, ctypes.c_float(0.0), 16, dummy, dummy, None) == 1
    assert lib.bsa_probe_fit(1, 1, 1, 128, dummy, dummy, dummy, 64, 1, ctypes.c_float(0.1), 17, dummy, dummy, None) == 4
    # tau count must be 1 or one per head
    assert lib.bsa_top_p_mask(dummy, 4, 8, 8, dummy, 3, 4, dummy, dummy, dummy, None) == 2
    # error-aware routing: block errors need bfloat16 and at most 4096 probes; routes at most
    # 1024 key clusters; null pointers
    f = ctypes.c_float(0.125)
    assert lib.bsa_block_error(1, 2, 2, 1024, 128, 0, dummy, 16, f, dummy, 1 << 30, dummy, 16, 1, dummy, dummy, dummy, dummy, 1 << 30, None) == 4
    assert lib.bsa_block_error(1, 2, 2, 1024, 128, 1, dummy, 4097, f, dummy, 1 << 30, dummy, 16, 1, dummy, dummy, dummy, dummy, 1 << 30, None) == 4
    assert lib.bsa_block_error(1, 3, 2, 1024, 128, 1, dummy, 16, f, dummy, 1 << 30, dummy, 16, 1, dummy, dummy, dummy, dummy, 1 << 30, None) == 2
    assert lib.bsa_block_error(1, 2, 2, 1024, 128, 1, dummy, 16, f, dummy, 16, dummy, 16, 1, dummy, dummy, dummy, dummy, 1 << 30, None) == 5
    assert lib.bsa_error_route(dummy, 4, 1025, dummy, 0, 10, dummy, dummy, dummy, None) == 4
    assert lib.bsa_error_route(None, 4, 16, dummy, 0, 10, dummy, dummy, dummy, None) == 1
    assert lib.bsa_query_centroids(1, 1, 1, 100, 96, 1, dummy, dummy, dummy, 4, 1, dummy, None) == 4


def test_workspace_sizes(lib):
    from block_sparse_attention_antidiagonal_amd import _lib

    assert _lib.size_query("bsa_cluster_layout_workspace_size", 1, 32760, 256) == 32 * 256 * 4
    assert _lib.size_query("bsa_cluster_layout_workspace_size", 40, 32760, 256) == 40 * 32 * 256 * 4
    nb, ns, ntk = 256, 2048, 8  # key tiles of 256 strided rows
    assert _lib.size_query("bsa_antidiag_scores_workspace_size", 1, 40, 40, 32760, 128, 128, 16) == \
        40 * ns * (nb + 2 * ntk) * 4
    assert _lib.size_query("bsa_probe_attention_workspace_size", 1, 40, 32760, 128, 64) == 40 * 17 * 64 * 130 * 4
    # packed K/V: per head ceil(S/64) + C token tiles and ceil(C/64) centroid tiles of 64 x D
    # keys and 64 x D values; sections (per-head format summary, tile flags, K, V, then per
    # layout the cluster tile offsets and the log2 of each centroid count) 256-byte aligned
    tiles = 40 * (512 + 256 + 4)
    tile_bytes = 64 * 128 * 2
    a = lambda n: -(-n // 256) * 256
    expect = 256 + a(tiles) + 2 * tiles * tile_bytes + a(257 * 4) + 256 * 4
    assert _lib.size_query("bsa_kv_pack_workspace_size", 1, 40, 32760, 128, 1, 256, 1) == expect
    expect40 = 256 + a(tiles) + 2 * tiles * tile_bytes + a(40 * 257 * 4) + 40 * 256 * 4
    assert _lib.size_query("bsa_kv_pack_workspace_size", 1, 40, 32760, 128, 1, 256, 40) == expect40
    with pytest.raises(RuntimeError):
        _lib.size_query("bsa_kv_pack_workspace_size", 1, 40, 32760, 128, 1, 256, 7)  # neither 1 nor B * Hkv
    # attention tile lists: per mask row one int32 per centroid or token tile, plus a count;
    # the work order and each unit's rank in its group (one int32 per batch x head x query
    # cluster each), one total per K/V group (sized for B x Hq groups), the queue counters, and
    # the staged correction of each (batch, query head): A^T as bfloat16 high and low parts in
    # rows of D + 8, then c (the largest of the bfloat16 and float32 forms at D = 128), in
    # whole kilobytes
    rows, stride = 40 * 256, 4 + 512 + 256
    units = 40 * 256
    image = -(-(2 * 128 * 136 * 2 + 128 * 4) // 1024) * 1024
    assert _lib.size_query("bsa_sparse_attention_workspace_size", 1, 40, 40, 256, 32760, 256) == \
        -(-rows * stride * 4 // 256) * 256 + (-(-rows * 4 // 256) * 256) + 2 * (-(-units * 4 // 256) * 256) + \
        (-(-40 * 4 // 256) * 256) + 256 + 40 * image


def test_block_error_workspace_size(lib):
    """The first pass's partial rows (24 chunks of 32 token tiles for S = 32760, 256 clusters),
    its rows and its log-sum-exp, each section 256-byte aligned."""
    from block_sparse_attention_antidiagonal_amd import _lib

    a = lambda n: -(-n // 256) * 256
    assert _lib.size_query("bsa_block_error_workspace_size", 1, 40, 40, 32760, 128, 256, 256) == \
        a(40 * 24 * 256 * 130 * 4) + a(40 * 256 * 128 * 4) + a(40 * 256 * 4)
    # packed probe rows: 24 token chunks plus the centroid chunk, dense and sparse rows
    assert _lib.size_query("bsa_probe_attention_packed_workspace_size", 1, 40, 40, 32760, 128, 64, 256) == \
        40 * 25 * 128 * 130 * 4


@pytest.mark.parametrize("grid,tile,window", [((1, 3, 4), (1, 1, 1), (1, 3, 3)), ((4, 8, 12), (2, 4, 4), (1, 2, 3)),
                                              ((5, 9, 10), (2, 4, 4), (3, 1, 3)), ((11, 4, 7), (1, 1, 1), (7, 3, 3))])
def test_sliding_tile_mask_host_helper(lib, grid, tile, window):
    """The host helper (C++) against the oracle, bit for bit."""
    from block_sparse_attention_antidiagonal_amd import api
    from oracle import static_masks as osm
    got = api.sliding_tile_block_mask(*grid, tile, window)
    assert np.array_equal(got, osm.sliding_tile_block_mask(*grid, tile, window))
