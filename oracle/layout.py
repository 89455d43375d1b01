"""Token layout: cluster-major order and sliding-tile labels (oracle).

[SPR] (group-major permutation paragraph): queries, keys and values are permuted into
group-major order before the sparse kernel and the output is written back.  Cluster
labels are caller inputs ([SBC] "Deviations from the papers": clusters are inputs).
"""

from __future__ import annotations

import numpy as np


def cluster_layout(labels: np.ndarray, C: int):
    """Group-major order of tokens.

    Returns (perm, offsets, counts): ``perm`` lists token positions cluster by cluster,
    keeping the given order inside a cluster (a stable sort by label); cluster ``c`` owns
    ``perm[offsets[c]:offsets[c+1]]`` and has ``counts[c]`` tokens.
    """
    labels = np.asarray(labels)
    if labels.size and (labels.min() < 0 or labels.max() >= C):
        raise ValueError("labels must lie in [0, C)")
    perm = np.argsort(labels, kind="stable").astype(np.int64)
    counts = np.bincount(labels, minlength=C).astype(np.int64)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets, counts


def tile_labels(T: int, H: int, W: int, tile, chunk: int = 0) -> np.ndarray:
    """Cluster labels of a T x H x W token grid in raster order ([SBC] API table, Recipe).

    Each token belongs to the sliding-tile 3-D tile of size ``tile`` = (tt, th, tw) that
    contains it; tiles are numbered in raster order, and edge tiles may be partial.
    ``chunk == 0`` returns the tile id.  ``chunk > 0`` ranks the tokens tile by tile
    (raster order inside a tile) and returns ``rank // chunk``: equal-size clusters that
    follow the tiles, for grids that no tile of ``chunk`` tokens divides.
    """
    tt, th, tw = tile
    ny = -(-H // th)
    nx = -(-W // tw)
    tile_id = np.empty(T * H * W, dtype=np.int64)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                tile_id[(t * H + y) * W + x] = ((t // tt) * ny + (y // th)) * nx + (x // tw)
    if chunk == 0:
        return tile_id.astype(np.int32)
    # Raster index increases with (t, y, x), so a stable sort by tile id gives tile-major
    # order with raster order inside each tile.
    order = np.argsort(tile_id, kind="stable")
    rank = np.empty_like(order)
    rank[order] = np.arange(order.size)
    return (rank // chunk).astype(np.int32)
