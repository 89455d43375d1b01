"""Per-row top-p block selection (oracle).

[HMR] "XAttention -- anti-diagonal block scoring": each query block keeps the smallest set
of key blocks whose mass reaches a fraction tau of its row total.  [HMR] "Deviations from
the papers": at least one block per row, and key block 0 is not forced.  [HMR] "Recipe":
tau is a scalar or one value per head.

Reading for equal scores: blocks are taken in descending score order, equal scores by
lower key-block index, so the kept set is unique.
"""

from __future__ import annotations

import numpy as np


def top_p_row(scores_row: np.ndarray, tau: float) -> np.ndarray:
    """Keep bits (uint8) for one row of block scores."""
    s = np.asarray(scores_row, dtype=np.float64)
    order = np.argsort(-s, kind="stable")  # descending, equal scores by lower index
    csum = np.cumsum(s[order])
    target = float(tau) * s.sum()
    reached = np.nonzero(csum >= target)[0]
    last = int(reached[0]) if reached.size else s.size - 1
    keep = np.zeros(s.size, dtype=np.uint8)
    keep[order[: last + 1]] = 1
    return keep


def top_p_block_mask(scores: np.ndarray, tau) -> np.ndarray:
    """Keep bits for a [..., nq, nk] score array; ``tau`` scalar or per leading head.

    ``scores`` is [H, nq, nk] (or [nq, nk]); ``tau`` is a scalar or an [H] array.
    """
    scores = np.asarray(scores, dtype=np.float64)
    squeeze = scores.ndim == 2
    if squeeze:
        scores = scores[None]
    H = scores.shape[0]
    taus = np.broadcast_to(np.asarray(tau, dtype=np.float64), (H,))
    keep = np.zeros(scores.shape, dtype=np.uint8)
    for h in range(H):
        for a in range(scores.shape[1]):
            keep[h, a] = top_p_row(scores[h, a], taus[h])
    return keep[0] if squeeze else keep


def kept_lists(keep: np.ndarray):
    """Ascending kept key blocks of each row: (counts [rows], list of index arrays)."""
    rows = keep.reshape(-1, keep.shape[-1])
    idx = [np.nonzero(r)[0] for r in rows]
    return np.array([len(i) for i in idx], dtype=np.int64), idx


def fragile_blocks(scores_row: np.ndarray, tau: float, eps_mass: float = 1e-5,
                   eps_tie: float = 1e-6) -> np.ndarray:
    """Blocks whose keep bit is decided within rounding of the cut (parity exclusion).

    A block is fragile when the cumulative mass before it lies within ``eps_mass`` of
    tau times the row total (so whether it is needed at all depends on rounding), or when
    it and its neighbour across the cut have scores within ``eps_tie`` (so their order
    can swap).  Returns a bool array.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    order = np.argsort(-s, kind="stable")
    sorted_s = s[order]
    csum = np.cumsum(sorted_s)
    excl = csum - sorted_s
    target = float(tau) * s.sum()
    fragile = np.zeros(s.size, dtype=bool)
    near = np.abs(excl - target) <= eps_mass
    fragile[order[near]] = True
    keep = top_p_row(s, tau)
    last = int(keep.sum()) - 1
    # Equal-ish scores straddling the cut can be ordered either way.
    lo = last
    while lo > 0 and abs(sorted_s[lo - 1] - sorted_s[last]) <= eps_tie:
        lo -= 1
    hi = last
    while hi + 1 < s.size and abs(sorted_s[hi + 1] - sorted_s[last]) <= eps_tie:
        hi += 1
    if hi > last:
        fragile[order[lo:hi + 1]] = True
    return fragile
