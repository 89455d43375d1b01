"""Pins for the oracle's static sliding-tile block masks (CPU only).

Hand-worked windows on a small grid, the row count every clamped window keeps, the
degenerate windows (one tile: identity; the whole grid: everything), symmetric
neighbourhoods away from the edges, and the page's consistency statement: the token-level
mask equals the tile-level mask expanded through the tile labels ([SBC] "Recipe: STA with
both repairs").
"""

import itertools

import numpy as np
import pytest

from oracle import layout as olay
from oracle import static_masks as osm


def test_hand_worked_windows():
    """Grid 1 x 3 x 4 tiles, window (1, 3, 3): every row covers all 3 rows of tiles; along x
    the windows are [0, 3) for x = 0, 1 and [1, 4) for x = 2, 3 (shifted inward at the edges)."""
    keep = osm.sliding_tile_block_mask(1, 3, 4, (1, 1, 1), (1, 3, 3))
    windows = {0: {0, 1, 2}, 1: {0, 1, 2}, 2: {1, 2, 3}, 3: {1, 2, 3}}
    for qy, qx, ky, kx in itertools.product(range(3), range(4), range(3), range(4)):
        assert keep[qy * 4 + qx, ky * 4 + kx] == (kx in windows[qx])


def test_window_start_values():
    assert [osm.window_start(a, 3, 7) for a in range(7)] == [0, 0, 1, 2, 3, 4, 4]
    assert [osm.window_start(a, 4, 7) for a in range(7)] == [0, 0, 0, 1, 2, 3, 3]
    assert [osm.window_start(a, 9, 5) for a in range(5)] == [0] * 5


@pytest.mark.parametrize("grid,window", [((3, 4, 5), (1, 3, 3)), ((5, 2, 6), (3, 5, 4)), ((2, 7, 3), (2, 2, 9))])
def test_rows_keep_the_full_window(grid, window):
    keep = osm.sliding_tile_block_mask(*grid, (1, 1, 1), window)
    expect = int(np.prod([min(w, n) for w, n in zip(window, grid)]))
    assert np.all(keep.sum(axis=1) == expect)


def test_degenerate_windows():
    assert np.array_equal(osm.sliding_tile_block_mask(2, 3, 4, (1, 1, 1), (1, 1, 1)), np.eye(24, dtype=np.uint8))
    assert np.all(osm.sliding_tile_block_mask(2, 3, 4, (1, 1, 1), (2, 3, 4)) == 1)
    assert np.all(osm.sliding_tile_block_mask(2, 3, 4, (1, 1, 1), (5, 9, 9)) == 1)


def test_interior_neighbourhoods_are_symmetric():
    n, w = 9, (3, 5, 3)
    keep = osm.sliding_tile_block_mask(n, n, n, (1, 1, 1), w)
    idx = lambda t, y, x: (t * n + y) * n + x
    for q in [(4, 4, 4), (3, 4, 5), (2, 2, 2)]:
        for k in itertools.product(range(n), repeat=3):
            inside = all(abs(k[i] - q[i]) <= w[i] // 2 for i in range(3))
            assert keep[idx(*q), idx(*k)] == inside


@pytest.mark.parametrize("T,H,W,tile,window", [(4, 8, 12, (2, 4, 4), (1, 2, 3)), (5, 9, 10, (2, 4, 4), (3, 1, 3)),
                                               (3, 6, 6, (1, 3, 2), (3, 3, 3))])
def test_token_mask_is_tile_mask_through_labels(T, H, W, tile, window):
    """The page's consistency statement, on divisible and ragged grids."""
    tok = osm.sliding_tile_block_mask(T, H, W, tile, window)
    nt, nh, nw = -(-T // tile[0]), -(-H // tile[1]), -(-W // tile[2])
    til = osm.sliding_tile_block_mask(nt, nh, nw, (1, 1, 1), window)
    lab = olay.tile_labels(T, H, W, tile)
    assert np.array_equal(tok, til[lab][:, lab])
