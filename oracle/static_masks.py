"""Static sliding-tile block masks (oracle; test infrastructure only).

[SBC] "Recipe: STA with both repairs": the block mask of sliding tile attention is built at
tile resolution, ``sliding_tile_block_mask(T // tt, H // th, W // tw, tile=(1, 1, 1),
window=window)``, and used with the clusters ``tile_labels(T, H, W, tile)``; expanding it
through the tile labels reproduces the token-level sliding-tile mask.  [HMR] "Static vs
dynamic masks": sliding-tile masks are fixed patterns that do not depend on the content.

Readings taken where the pages are silent:
  * The function takes a grid of nT x nH x nW cells in raster order, grouped into tiles of
    ``tile`` cells (edge tiles partial), and returns the [N, N] keep matrix over the cells
    (N = nT nH nW): cell i attends cell j when j's tile lies in the window of i's tile.  With
    tile = (1, 1, 1) the cells are the tiles themselves and the result is the cluster-level
    mask; with the real tile size on the token grid it is the token-level mask.
  * ``window`` = (wt, wh, ww) counts tiles.  Along each axis the window of a query tile at
    coordinate a starts at a - w // 2, shifted inward at the edges so that it stays inside
    the n tiles of that axis: start = min(max(a - w // 2, 0), max(n - w, 0)).  Every query
    tile therefore keeps exactly prod(min(w, n)) key tiles (the window slides rather than
    shrinks), the usual boundary rule of sliding-window attention on a grid.
"""

from __future__ import annotations

import numpy as np


def window_start(a: int, w: int, n: int) -> int:
    """First tile of the window of width w around coordinate a on an axis of n tiles."""
    return min(max(a - w // 2, 0), max(n - w, 0))


def _tile_coords(n_cells, tile):
    """Tile coordinates (raster order of cells) and tile counts per axis."""
    nT, nH, nW = n_cells
    tt, th, tw = tile
    t = np.repeat(np.arange(nT), nH * nW) // tt
    y = np.tile(np.repeat(np.arange(nH), nW), nT) // th
    x = np.tile(np.arange(nW), nT * nH) // tw
    counts = (-(-nT // tt), -(-nH // th), -(-nW // tw))
    return (t, y, x), counts


def sliding_tile_block_mask(nT: int, nH: int, nW: int, tile=(1, 1, 1), window=(1, 1, 1)) -> np.ndarray:
    """Keep bits uint8 [N, N] over the cells of an nT x nH x nW raster grid (see the header)."""
    coords, counts = _tile_coords((nT, nH, nW), tile)
    N = nT * nH * nW
    keep = np.ones((N, N), dtype=bool)
    for axis in range(3):
        a = coords[axis]
        w, n = int(window[axis]), counts[axis]
        start = np.array([window_start(int(v), w, n) for v in a])
        inside = (a[None, :] >= start[:, None]) & (a[None, :] < start[:, None] + w)
        keep &= inside
    return keep.astype(np.uint8)
