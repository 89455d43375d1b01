"""The whole path for one (batch, head), composed from the oracle's stages.

Order of stages ([HMR] "Recipe"; [SBC] "Recipe: STA with both repairs"; [SPR] timing
paragraph): cluster layout -> block scores -> top-p mask -> compensated (or hard-drop)
block-sparse attention -> exact probe rows -> ridge fit -> correction on every row.

Inputs are duck-typed workload objects with fields q, k, v ([B, H, S, D]), labels, C,
scale, mask_mode ("given" / "scored"), mask, block, stride, score_scale, tau, pool_gqa,
compensate, probes, lam, rank, Hq, Hkv.
"""

from __future__ import annotations

import numpy as np

from .attention import compensated_attention, dense_attention_rows
from .layout import cluster_layout
from .repair import apply_correction, ridge_fit, select_probe_rows
from .scoring import antidiagonal_block_scores
from .topp import top_p_block_mask


def head_scores(wl, b: int, hq: int) -> np.ndarray:
    """Normalized antidiagonal block scores of query head hq (cluster-major order)."""
    perm, _, counts = cluster_layout(wl.labels, wl.C)
    kvh = hq // (wl.Hq // wl.Hkv)
    return antidiagonal_block_scores(wl.q[b, hq], wl.k[b, kvh], perm, wl.block, wl.stride, wl.score_scale)


def mask_scores(wl, b: int, hm: int) -> np.ndarray:
    """Scores that decide mask head hm: the head's own, or its group's mean (shared routes)."""
    if wl.pool_gqa:
        g = wl.Hq // wl.Hkv
        return np.mean([head_scores(wl, b, h) for h in range(hm * g, (hm + 1) * g)], axis=0)
    return head_scores(wl, b, hm)


def check_scored_layout(wl) -> None:
    """Scored masks index clusters by block: every cluster is one block of the
    cluster-major order, i.e. all clusters hold ``block`` tokens except possibly the last."""
    _, _, counts = cluster_layout(wl.labels, wl.C)
    nb = -(-wl.labels.size // wl.block)
    if wl.C != nb or np.any(counts[:-1] != wl.block) or counts[-1] < 1 or counts[-1] > wl.block:
        raise ValueError("scored masks need clusters that are the blocks of the cluster-major order")


def head_mask(wl, b: int, hm: int, scores=None) -> np.ndarray:
    """Keep bits [C, C] of mask head hm of batch entry b."""
    if wl.mask_mode == "given":
        m = wl.mask
        return m[b if m.shape[0] > 1 else 0, hm if m.shape[1] > 1 else 0]
    check_scored_layout(wl)
    if scores is None:
        scores = mask_scores(wl, b, hm)
    return top_p_block_mask(scores, float(wl.tau[hm]))


def mask_head_of(wl, hq: int) -> int:
    """Which mask a query head uses: its own, its K/V group's, or the shared one."""
    if wl.mask_mode == "given":
        Hm = wl.mask.shape[1]
    else:
        Hm = wl.Hkv if wl.pool_gqa else wl.Hq
    if Hm == 1:
        return 0
    if Hm == wl.Hq:
        return hq
    return hq // (wl.Hq // Hm)


def run_head(wl, b: int, hq: int, rows=None, keep=None, probe_idx=None, weights=None) -> dict:
    """Run the path for query head hq of batch entry b.

    ``rows`` selects the output rows to return (default all).  ``keep`` overrides the mask
    (so attention can be checked on the exact mask another implementation chose);
    ``probe_idx``/``weights`` override the probe selection.
    """
    kvh = hq // (wl.Hq // wl.Hkv)
    q, k, v = wl.q[b, hq], wl.k[b, kvh], wl.v[b, kvh]
    S = q.shape[0]
    if keep is None:
        keep = head_mask(wl, b, mask_head_of(wl, hq))
    rows = np.arange(S) if rows is None else np.asarray(rows)
    res = dict(keep=keep, rows=rows)
    if wl.probes:
        if probe_idx is None:
            probe_idx, weights = select_probe_rows(wl.labels, wl.C, wl.probes)
        need = np.concatenate([rows, probe_idx])
    else:
        need = rows
    out, lse = compensated_attention(q, k, v, wl.labels, wl.labels, keep, wl.scale, wl.compensate, rows=need)
    res["out_sparse"] = out[: rows.size]
    res["lse"] = lse[: rows.size]
    if wl.probes:
        o_s_p = out[rows.size:]
        o_d_p = dense_attention_rows(q[probe_idx], k, v, wl.scale)
        fit = ridge_fit(o_s_p, o_d_p, weights, wl.lam, wl.rank)
        res.update(probe_idx=probe_idx, weights=weights, o_sparse_p=o_s_p, o_dense_p=o_d_p, fit=fit)
        res["out"] = apply_correction(res["out_sparse"], fit["A"], fit["c"])
    else:
        res["out"] = res["out_sparse"]
    return res
