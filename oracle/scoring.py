"""XAttention antidiagonal block scores (oracle).

[HMR] "XAttention -- anti-diagonal block scoring": each stride x stride sub-block of Q K^T
is summarized by the sum along its anti-diagonal; the strided logits are softmaxed per
row, summed per block x block tile, and ([HMR] "Deviations from the papers") each row of
block scores is divided by its total.  Padding ([HMR] "Out of scope, and why"): the
sequence is zero-padded to a multiple of the block size, and padded keys still take
softmax mass.

Readings taken where the page is silent:
  * the strided logit is ``score_scale`` times the anti-diagonal sum (the page gives no
    temperature; the default score_scale is the attention scale D^-1/2);
  * scoring runs on the cluster-major token order given by ``perm`` (identity when the
    labels are already ``arange(S) // block``), so block a of the scores is cluster a;
  * grouped-query masks score every query head and average the normalized block scores of
    the heads sharing one K/V head.
"""

from __future__ import annotations

import numpy as np


def strided_logits(q: np.ndarray, k: np.ndarray, stride: int, score_scale: float) -> np.ndarray:
    """Anti-diagonal sums of every stride x stride sub-block of q k^T, times score_scale.

    q, k: [N, D] with N a multiple of ``stride``.  Entry (i', j') sums q[i's + s-1-t] .
    k[j's + t] over t = 0..s-1: the sub-block's anti-diagonal, whose row and column offsets
    add up to s-1.  Written as one product: strided query row i' lists its s tokens in
    reverse order, strided key row j' in forward order, so their dot product pairs exactly
    the anti-diagonal elements.
    """
    N, D = q.shape
    n = N // stride
    q_rev = q.reshape(n, stride, D)[:, ::-1, :].reshape(n, stride * D)
    k_fwd = k.reshape(n, stride, D).reshape(n, stride * D)
    return score_scale * (q_rev @ k_fwd.T)


def antidiagonal_block_scores(q: np.ndarray, k: np.ndarray, perm, block: int, stride: int,
                              score_scale: float) -> np.ndarray:
    """Normalized block scores [nb, nb] for one head.

    q, k: [S, D] in the caller's token order; perm: cluster-major order (None = identity).
    """
    if block % stride != 0:
        raise ValueError("block must be a multiple of stride")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if perm is not None:
        q = q[perm]
        k = k[perm]
    S, D = q.shape
    nb = -(-S // block)
    s_pad = nb * block
    qp = np.zeros((s_pad, D))
    kp = np.zeros((s_pad, D))
    qp[:S] = q
    kp[:S] = k
    logits = strided_logits(qp, kp, stride, score_scale)
    # Row softmax over every strided key column, padded ones included.
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    r = block // stride
    mass = p.reshape(nb, r, nb, r).sum(axis=(1, 3))
    return mass / mass.sum(axis=1, keepdims=True)


def pooled_group_scores(scores_per_head: np.ndarray, group: int) -> np.ndarray:
    """Average normalized scores over the query heads of each K/V group.

    scores_per_head: [Hq, nb, nb] -> [Hq // group, nb, nb].
    """
    Hq = scores_per_head.shape[0]
    return scores_per_head.reshape(Hq // group, group, *scores_per_head.shape[1:]).mean(axis=1)
