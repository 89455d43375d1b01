"""Block-sparse video-DiT attention for AMD Instinct MI355X (gfx950).

Antidiagonal block scoring, per-row top-p block masks, block-sparse flash attention with
centroid compensation, probe-fitted residual repair, head-wise reuse of block masks across
calls (pooled Q/K drift with a layer gate) and error-aware block routing (query-centroid
probes, per-block compensation error, error-to-cost routes), as hand-written HIP kernels
behind a C ABI (include/bsa.h, libbsa.so).  This package is the thin Python binding:
importing it loads libbsa.so and fails if the library has not been built.
"""

from . import _lib

_lib.load()

from .api import (  # noqa: E402,F401
    BlockMask,
    ClusterLayout,
    HeadMaskCache,
    PackedKV,
    antidiagonal_block_scores,
    block_error,
    block_sparse_attention,
    block_sparse_attention_noalloc,
    centroid_compensated_attention,
    centroids,
    cluster_layout,
    correct,
    error_route,
    gather_rows,
    kv_pack,
    kmeans,
    kv_pack_centroids,
    mask_from_keep,
    mask_reuse_decide,
    mask_reuse_update,
    probe_apply,
    probe_attention,
    probe_attention_packed,
    probe_fit,
    pooled_qk,
    query_centroids,
    response_partition,
    select_probe_rows,
    select_probe_rows_layouts,
    sliding_tile_block_mask,
    tile_labels,
    top_p_block_mask,
)
from .path import PathConfig, PathResult, SparseAttentionPath  # noqa: E402,F401
