"""Head-wise temporal mask reuse (oracle; test infrastructure only).

[HMR] "HEART -- head-wise temporal mask reuse", Temporal Mask Reuse: each head keeps an
anchor, the token means of Q and K at the step where its mask was last built, together with
that mask.  At a later step the head's drift is the L1 distance between the anchor's means
and the current ones, summed over Q and K.  A drift above a global threshold delta rebuilds
the head's mask and moves its anchor; otherwise the cached mask is used again.  A
layer-level override refreshes no head when fewer than 40% of the layer's heads ask for a
refresh, and every head when more than 80% do.
[HMR] "What mlx-arsenal ships": the pooled summary and the L1 drift (optionally relative)
are separate functions; the cache works in two phases (decide which heads refresh, then
store the new masks and anchors) and the layer gate is optional.
[HMR] "Recipe": the first call refreshes every head; heads that refresh take the newly
predicted mask, the others keep theirs.
[HMR] "Deviations from the papers": the relative drift divides by the anchor's L1 norm.

Readings taken where the page is silent or leaves a choice:
  * A mask head's summary is the token mean of the queries and of the keys its mask serves.
    One mask per query head (Hm = Hq): that head's Q and its K/V head's K.  One mask per K/V
    group (Hm = Hkv): Q averaged over the group's query heads and all tokens, and the
    group's K.  One mask for all heads (Hm = 1): Q over all query heads, K over all K/V heads.
  * Relative drift: the summed L1 distance divided by the L1 norm of the whole anchor,
    ||q_a||_1 + ||k_a||_1.  A zero anchor norm gives 0 when nothing moved and +inf otherwise.
  * A head asks for a refresh when its drift is strictly greater than delta.
  * "Fewer than 40%" and "more than 80%" are strict: at exactly 40% or 80% the per-head
    decisions stand.
  * The gate counts the Hm mask heads of one batch entry (the page keeps one cache per layer
    and per guidance branch; a batch entry plays the role of one such cache).
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

GATE_LOW = 0.4   # fewer than this fraction asking: no head refreshes
GATE_HIGH = 0.8  # more than this fraction asking: every head refreshes


def pooled_summary(q: np.ndarray, k: np.ndarray, Hm: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token means (float64) of the queries and keys each mask head serves.

    q: [B, Hq, S, D], k: [B, Hkv, S, D]; Hm in {Hq, Hkv, 1}.  Returns qbar, kbar [B, Hm, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qh = q.mean(axis=2)  # [B, Hq, D]: the mean over tokens of each query head
    kh = k.mean(axis=2)  # [B, Hkv, D]
    if Hm == Hq:
        return qh, kh[:, np.arange(Hq) // G]
    if Hm == Hkv:
        return qh.reshape(B, Hkv, G, D).mean(axis=2), kh
    if Hm == 1:
        return qh.mean(axis=1, keepdims=True), kh.mean(axis=1, keepdims=True)
    raise ValueError("Hm must be Hq, Hkv or 1")


def l1_drift(qbar, kbar, anchor_q, anchor_k, relative: bool = False) -> np.ndarray:
    """Drift of every mask head: ||qbar - q_a||_1 + ||kbar - k_a||_1 over the last axis,
    divided by ||q_a||_1 + ||k_a||_1 when ``relative``."""
    qbar, kbar = np.asarray(qbar, np.float64), np.asarray(kbar, np.float64)
    anchor_q, anchor_k = np.asarray(anchor_q, np.float64), np.asarray(anchor_k, np.float64)
    d = np.abs(qbar - anchor_q).sum(axis=-1) + np.abs(kbar - anchor_k).sum(axis=-1)
    if not relative:
        return d
    norm = np.abs(anchor_q).sum(axis=-1) + np.abs(anchor_k).sum(axis=-1)
    out = np.empty_like(d)
    pos = norm > 0
    out[pos] = d[pos] / norm[pos]
    out[~pos] = np.where(d[~pos] > 0, np.inf, 0.0)
    return out


def layer_gate(want: np.ndarray) -> np.ndarray:
    """Apply the layer override to per-head requests want [B, Hm] (bool), per batch entry."""
    want = np.asarray(want, dtype=bool)
    out = want.copy()
    for b in range(want.shape[0]):
        frac = want[b].sum() / want.shape[1]
        if frac < GATE_LOW:
            out[b] = False
        elif frac > GATE_HIGH:
            out[b] = True
    return out


def refresh_decision(drift: np.ndarray, delta: float, have_anchor: bool, gate: bool = True) -> np.ndarray:
    """Which mask heads refresh: all of them without an anchor (the first call), else
    drift > delta, passed through the layer gate when ``gate``."""
    drift = np.asarray(drift, dtype=np.float64)
    if not have_anchor:
        return np.ones(drift.shape, dtype=bool)
    want = drift > delta
    return layer_gate(want) if gate else want


class HeadMaskCache:
    """Per-head masks with their anchors, in two phases per step.

    should_refresh() computes the current summaries and decides which heads refresh;
    update() stores the new masks and moves the anchors of exactly those heads and returns
    the mask to attend with (new rows where refreshed, cached rows elsewhere).  Masks are
    keep bits [B, Hm, Cq, Ck].
    """

    def __init__(self, delta: float, relative: bool = False, gate: bool = True):
        self.delta = float(delta)
        self.relative = bool(relative)
        self.gate = bool(gate)
        self.anchor_q: Optional[np.ndarray] = None
        self.anchor_k: Optional[np.ndarray] = None
        self.mask: Optional[np.ndarray] = None
        self._cur: Optional[Tuple[np.ndarray, np.ndarray]] = None
        self.last_drift: Optional[np.ndarray] = None

    def should_refresh_summary(self, qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
        """Decision from given summaries qbar, kbar [B, Hm, D]."""
        qbar, kbar = np.asarray(qbar, np.float64), np.asarray(kbar, np.float64)
        self._cur = (qbar, kbar)
        have = self.anchor_q is not None
        if have:
            self.last_drift = l1_drift(qbar, kbar, self.anchor_q, self.anchor_k, self.relative)
        else:
            self.last_drift = np.zeros(qbar.shape[:2])
        return refresh_decision(self.last_drift, self.delta, have, self.gate)

    def should_refresh(self, q: np.ndarray, k: np.ndarray, Hm: int) -> np.ndarray:
        return self.should_refresh_summary(*pooled_summary(q, k, Hm))

    def update(self, new_mask: np.ndarray, refresh: np.ndarray) -> np.ndarray:
        if self._cur is None:
            raise RuntimeError("update() needs a preceding should_refresh()")
        refresh = np.asarray(refresh, dtype=bool)
        qbar, kbar = self._cur
        new_mask = np.asarray(new_mask)
        if self.mask is None:
            if not refresh.all():
                raise ValueError("the first update must refresh every head")
            self.mask = new_mask.copy()
            self.anchor_q, self.anchor_k = qbar.copy(), kbar.copy()
        else:
            self.mask[refresh] = new_mask[refresh]
            self.anchor_q[refresh] = qbar[refresh]
            self.anchor_k[refresh] = kbar[refresh]
        self._cur = None
        return self.mask.copy()
