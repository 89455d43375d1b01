"""Pins for the oracle's head-wise mask reuse (CPU only).

The page prints no worked example for mask reuse, so the oracle is pinned by closed forms
(means of ramps, L1 distances of shifted vectors), brute-force loops over tokens on tiny
inputs, hand-worked gate decisions at and around the 40% / 80% thresholds, and a scripted
five-step scenario whose refresh decisions, cached masks and anchors were worked out by hand
from the rules in [HMR] "HEART -- head-wise temporal mask reuse" (expected values written
below as literals).
"""

import numpy as np
import pytest

from oracle import reuse as orr


# ---------------------------------------------------------------- pooled summary

def _ramp(B, H, S, D, head_step, dim_step):
    i = np.arange(S)[None, None, :, None]
    h = np.arange(H)[None, :, None, None]
    d = np.arange(D)[None, None, None, :]
    b = np.arange(B)[:, None, None, None]
    return (i + head_step * h + dim_step * d + 1000.0 * b) * np.ones((B, H, S, D))


@pytest.mark.parametrize("Hm_kind", ["Hq", "Hkv", "one"])
def test_pooled_summary_ramp_closed_form(Hm_kind):
    B, Hq, Hkv, S, D = 2, 6, 3, 7, 4
    G = Hq // Hkv
    q = _ramp(B, Hq, S, D, 10.0, 100.0)
    k = _ramp(B, Hkv, S, D, 20.0, 300.0)
    Hm = {"Hq": Hq, "Hkv": Hkv, "one": 1}[Hm_kind]
    qbar, kbar = orr.pooled_summary(q, k, Hm)
    mid = (S - 1) / 2.0  # mean of 0..S-1
    d = np.arange(D)
    for b in range(B):
        for m in range(Hm):
            if Hm == Hq:
                qh, kh = [m], [m // G]
            elif Hm == Hkv:
                qh, kh = list(range(m * G, (m + 1) * G)), [m]
            else:
                qh, kh = list(range(Hq)), list(range(Hkv))
            np.testing.assert_allclose(qbar[b, m], mid + 10.0 * np.mean(qh) + 100.0 * d + 1000.0 * b, rtol=1e-14)
            np.testing.assert_allclose(kbar[b, m], mid + 20.0 * np.mean(kh) + 300.0 * d + 1000.0 * b, rtol=1e-14)


def test_pooled_summary_brute_force():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, S, D = 1, 4, 2, 5, 3
    q = rng.standard_normal((B, Hq, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    qbar, kbar = orr.pooled_summary(q, k, Hkv)
    for g in range(Hkv):
        for d in range(D):
            acc = 0.0
            for h in (2 * g, 2 * g + 1):
                for i in range(S):
                    acc += q[0, h, i, d]
            assert abs(qbar[0, g, d] - acc / (2 * S)) < 1e-14
            acc = 0.0
            for i in range(S):
                acc += k[0, g, i, d]
            assert abs(kbar[0, g, d] - acc / S) < 1e-14


def test_pooled_summary_rejects_other_mask_heads():
    with pytest.raises(ValueError):
        orr.pooled_summary(np.zeros((1, 4, 2, 2)), np.zeros((1, 2, 2, 2)), 3)


# ---------------------------------------------------------------- drift

def test_drift_closed_forms():
    rng = np.random.default_rng(1)
    qa, ka = rng.standard_normal((2, 3, 8)), rng.standard_normal((2, 3, 8))
    assert np.all(orr.l1_drift(qa, ka, qa, ka) == 0.0)
    # shifting every component of q by c and of k by -e moves the drift to D(|c| + |e|)
    np.testing.assert_allclose(orr.l1_drift(qa + 0.25, ka - 1.5, qa, ka), 8 * (0.25 + 1.5), rtol=1e-14)


def test_relative_drift_hand_example():
    # anchor q = (1, -2), k = (3, 0): L1 norm 6; current q = (2, -2), k = (3, 1): distance 2
    d = orr.l1_drift([[2.0, -2.0]], [[3.0, 1.0]], [[1.0, -2.0]], [[3.0, 0.0]], relative=True)
    assert d.shape == (1,) and abs(d[0] - 1.0 / 3.0) < 1e-15
    raw = orr.l1_drift([[2.0, -2.0]], [[3.0, 1.0]], [[1.0, -2.0]], [[3.0, 0.0]])
    assert raw[0] == 2.0


def test_relative_drift_scale_invariant_and_zero_anchor():
    rng = np.random.default_rng(2)
    q, k, qa, ka = (rng.standard_normal((4, 16)) for _ in range(4))
    a = orr.l1_drift(q, k, qa, ka, relative=True)
    b = orr.l1_drift(7.0 * q, 7.0 * k, 7.0 * qa, 7.0 * ka, relative=True)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    z = np.zeros((2, 3))
    d = orr.l1_drift(np.array([[0.0, 0, 0], [0, 1.0, 0]]), z, z, z, relative=True)
    assert d[0] == 0.0 and d[1] == np.inf


# ---------------------------------------------------------------- gate and decision

@pytest.mark.parametrize("want,expect", [
    ([1, 0, 0, 0, 0], [0, 0, 0, 0, 0]),   # 20% < 40%: nobody refreshes
    ([1, 1, 0, 0, 0], [1, 1, 0, 0, 0]),   # exactly 40%: per-head decisions stand
    ([0, 1, 1, 1, 0], [0, 1, 1, 1, 0]),   # 60%
    ([1, 1, 1, 1, 0], [1, 1, 1, 1, 0]),   # exactly 80%: per-head decisions stand
    ([1, 1, 1, 1, 1], [1, 1, 1, 1, 1]),
    ([0, 0, 0, 0, 0], [0, 0, 0, 0, 0]),
    ([1, 1, 1, 1, 1, 1, 1, 1, 1, 0], [1] * 10),  # 90% > 80%: every head refreshes
    ([1, 1, 1, 0, 0, 0, 0, 0, 0, 0], [0] * 10),  # 30% < 40%
])
def test_layer_gate(want, expect):
    got = orr.layer_gate(np.array([want], dtype=bool))
    assert got.tolist() == [[bool(x) for x in expect]]


def test_gate_is_per_batch_entry():
    want = np.array([[1, 0, 0, 0, 0], [1, 1, 1, 1, 1]], dtype=bool)
    assert orr.layer_gate(want).tolist() == [[False] * 5, [True] * 5]


def test_decision_threshold_is_strict_and_first_call_refreshes_all():
    assert orr.refresh_decision(np.array([[1.0, 1.0000001]]), 1.0, True, gate=False).tolist() == [[False, True]]
    assert orr.refresh_decision(np.zeros((2, 3)), 100.0, False).all()


# ---------------------------------------------------------------- the cache over a scripted sequence

def test_cache_scripted_sequence():
    """Five mask heads, D = 2, delta = 1, gate on.  Anchor summaries at step 0 are
    q_a[h] = (h, 0), k_a[h] = (0, h).  Each step's mask marks every entry with step + 1, so
    the cached mask shows which step built each head's mask."""
    H = 5
    cache = orr.HeadMaskCache(delta=1.0, relative=False, gate=True)

    def summ(qs, ks):
        return np.array([qs], dtype=np.float64), np.array([ks], dtype=np.float64)

    def step(qs, ks, marker):
        refresh = cache.should_refresh_summary(*summ(qs, ks))
        new = np.full((1, H, 2, 3), marker, dtype=np.uint8)
        return refresh, cache.update(new, refresh)

    q0 = [[h, 0.0] for h in range(H)]
    k0 = [[0.0, h] for h in range(H)]
    # step 0: no anchor yet, every head refreshes
    r, m = step(q0, k0, 1)
    assert r.tolist() == [[True] * H] and np.all(m == 1)
    # step 1: only head 0 drifts past delta (1.5 > 1); 1 of 5 = 20% < 40% -> nobody refreshes
    # (all values are dyadic, so every drift below is exact in binary floating point)
    q1 = [[0 + 1.5, 0.0]] + [[h + 0.25, 0.0] for h in range(1, H)]
    r, m = step(q1, k0, 2)
    assert cache.last_drift.tolist() == [[1.5, 0.25, 0.25, 0.25, 0.25]]
    assert r.tolist() == [[False] * H] and np.all(m == 1)
    # step 2: drifts 2, 1.25, 0.5, 0.125, 0 against the step-0 anchors; 2 of 5 = 40% -> per head
    q2 = [[2.0, 0.0], [2.25, 0.0], [2.5, 0.0], [3.125, 0.0], [4.0, 0.0]]
    r, m = step(q2, k0, 3)
    assert cache.last_drift.tolist() == [[2.0, 1.25, 0.5, 0.125, 0.0]]
    assert r.tolist() == [[True, True, False, False, False]]
    assert [int(m[0, h, 0, 0]) for h in range(H)] == [3, 3, 1, 1, 1]
    assert cache.anchor_q[0].tolist() == [[2.0, 0.0], [2.25, 0.0], [2.0, 0.0], [3.0, 0.0], [4.0, 0.0]]
    # step 3: head 0 moves k by (0, -1.5) from its anchor (0, 0); head 1 moves q to (4.25, 0)
    # from (2.25, 0); heads 2 and 3 move q by 2; head 4 stays: 4 of 5 = 80% -> per head
    q3 = [[2.0, 0.0], [4.25, 0.0], [4.0, 0.0], [3.0, 2.0], [4.0, 0.0]]
    k3 = [[0.0, -1.5], [0.0, 1.0], [0.0, 2.0], [0.0, 3.0], [0.0, 4.0]]
    r, m = step(q3, k3, 4)
    assert cache.last_drift.tolist() == [[1.5, 2.0, 2.0, 2.0, 0.0]]
    assert r.tolist() == [[True, True, True, True, False]]
    assert [int(m[0, h, 0, 0]) for h in range(H)] == [4, 4, 4, 4, 1]
    # step 4: exactly delta for every head (strict test: nobody asks), then one step where all
    # five drift by 5 -> 100% > 80%, all refresh
    q4 = [[q3[h][0] + 1.0, q3[h][1]] for h in range(4)] + [[5.0, 0.0]]
    r, m = step(q4, k3, 5)
    assert r.tolist() == [[False] * H] and [int(m[0, h, 0, 0]) for h in range(H)] == [4, 4, 4, 4, 1]
    q5 = [[v[0] + 5.0, v[1]] for v in q4]
    r, m = step(q5, k3, 6)
    assert r.tolist() == [[True] * H] and np.all(m == 6)


def test_cache_first_update_must_refresh_all():
    cache = orr.HeadMaskCache(delta=1.0)
    cache.should_refresh_summary(np.zeros((1, 2, 2)), np.zeros((1, 2, 2)))
    with pytest.raises(ValueError):
        cache.update(np.zeros((1, 2, 1, 1), np.uint8), np.array([[True, False]]))
    with pytest.raises(RuntimeError):
        orr.HeadMaskCache(delta=1.0).update(np.zeros((1, 1, 1, 1)), np.array([[True]]))


def test_cache_from_tokens_matches_summaries():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 6, 3))
    k = rng.standard_normal((1, 2, 6, 3))
    c1, c2 = orr.HeadMaskCache(0.5), orr.HeadMaskCache(0.5)
    r1 = c1.should_refresh(q, k, 4)
    r2 = c2.should_refresh_summary(*orr.pooled_summary(q, k, 4))
    assert r1.tolist() == r2.tolist() == [[True] * 4]
