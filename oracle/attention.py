"""Block-sparse attention with centroid compensation, and dense rows (oracle).

[SBC] "The problem": queries and keys are grouped into clusters; only kept (query cluster,
key cluster) blocks are computed; under hard drop the softmax is renormalized over the
kept keys.  [SBC] "SVG-EAR -- centroid compensation": every skipped key cluster c adds one
term with logit q_i . kbar_c . scale + log n_c and value vbar_c to the same softmax.
[SBC] "No LSE needed": the compensated output equals one softmax attention over the
extended keys [K; Kbar] and values [V; Vbar] with an additive mask that is 0 / -inf on
token columns (kept / skipped block) and log n_c / -inf on centroid columns (skipped /
kept block).  This module computes exactly that extended-key definition, one chunk of
query rows at a time (rows are independent), in float64.

Reading for a row whose every column is -inf (possible only under hard drop with an
all-skipped row): the output row is 0 and its log-sum-exp is -inf.
"""

from __future__ import annotations

import numpy as np

from .centroids import centroids


def compensated_attention(q, k, v, q_labels, k_labels, keep, scale: float, compensate: bool,
                          rows=None, chunk: int = 512, kbar=None, vbar=None, counts=None):
    """Output rows of block-sparse attention for one head.

    q: [Sq, D]; k, v: [Sk, D]; q_labels [Sq] in [0, Cq); k_labels [Sk] in [0, Ck);
    keep: [Cq, Ck] (nonzero = kept block).  ``compensate`` adds the centroid columns;
    otherwise skipped blocks are dropped.  ``rows`` selects query rows (default: all).
    ``kbar``, ``vbar`` [Ck, D] and ``counts`` [Ck]: centroid columns given by the caller (the
    page's API takes them as inputs); by default the clusters' means and sizes.
    Returns (out [len(rows), D], lse [len(rows)]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    keep = np.asarray(keep) != 0
    Ck = keep.shape[1]
    if kbar is None:
        kbar, vbar, n = centroids(k, v, k_labels, Ck)
    else:
        kbar = np.asarray(kbar, dtype=np.float64)
        vbar = np.asarray(vbar, dtype=np.float64)
        n = np.asarray(counts, dtype=np.int64)
    with np.errstate(divide="ignore"):
        log_n = np.log(n.astype(np.float64))  # log 0 = -inf: an empty cluster adds nothing
    k_ext = np.concatenate([k, kbar], axis=0)
    v_ext = np.concatenate([v, vbar], axis=0)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    for start in range(0, rows.size, chunk):
        r = rows[start:start + chunk]
        kept_blocks = keep[q_labels[r]]  # [r, Ck]
        token_bias = np.where(kept_blocks[:, k_labels], 0.0, -np.inf)  # [r, Sk]
        if compensate:
            centroid_bias = np.where(kept_blocks, -np.inf, log_n[None, :])  # [r, Ck]
        else:
            centroid_bias = np.full(kept_blocks.shape, -np.inf)
        logits = (q[r] @ k_ext.T) * scale + np.concatenate([token_bias, centroid_bias], axis=1)
        m = logits.max(axis=1)
        live = np.isfinite(m)
        e = np.zeros_like(logits)
        e[live] = np.exp(logits[live] - m[live, None])
        l = e.sum(axis=1)
        out[start:start + r.size][live] = (e[live] @ v_ext) / l[live, None]
        lse[start:start + r.size][live] = m[live] + np.log(l[live])
    return out, lse


def dense_attention_rows(q_rows, k, v, scale: float):
    """Exact dense softmax attention for the given query rows: softmax(q K^T scale) V."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = (q_rows @ k.T) * scale
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)
