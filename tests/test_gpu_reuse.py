"""GPU parity of head-wise temporal mask reuse against the oracle (oracle/reuse.py).

Pooled summaries: the kernel sums in float32 (per thread up to 128 rows, then 16 or 32 row
slots, then the chunks of 2048 rows, then the heads of a mask head), so its worst-case
absolute error is below (128 + 32 + nchunk + G) * 2^-24 * mean|x| per component (< 1e-5
mean|x|); the tests allow 2e-5 * mean|x| at S <= 4096 and 1e-4 * mean|x| at S = 32760.  Drifts are float32 sums
of 2D terms: relative error below 2D * 2^-24 plus the summaries' error.  Refresh decisions
are integers decided by floating point: the thresholds are placed midway between
consecutive oracle drifts, far from every drift, so both sides decide the same way; then
the flags must match exactly.  Cache updates and the head filter of the scorer are copies
and must match bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import reuse as orr
from synthetic.workloads import make_config, make_custom
from tests.gpu_common import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_antidiagonal_amd as m
    return m


def _summary_tol(x: np.ndarray, S: int) -> float:
    return (2e-5 if S <= 4096 else 1e-4) * float(np.mean(np.abs(x))) + 1e-7


@pytest.mark.parametrize("dtype,D,Hq,Hkv,S", [("bf16", 128, 4, 2, 1000), ("f32", 64, 4, 4, 1537),
                                              ("bf16", 64, 6, 3, 513), ("f32", 128, 2, 1, 511)])
@pytest.mark.parametrize("Hm_kind", ["Hq", "Hkv", "one"])
def test_pooled_qk(bsa, dtype, D, Hq, Hkv, S, Hm_kind):
    wl = make_custom(71 + S + D, B=2, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype=dtype, block=128)
    Hm = {"Hq": Hq, "Hkv": Hkv, "one": 1}[Hm_kind]
    say(f"pooled_qk {dtype} D={D} Hq={Hq} Hkv={Hkv} S={S} Hm={Hm}")
    qbar, kbar = bsa.api.pooled_qk(dev(wl.q, dtype), dev(wl.k, dtype), Hm)
    torch.cuda.synchronize()
    rq, rk = orr.pooled_summary(wl.q, wl.k, Hm)
    assert np.max(np.abs(host(qbar) - rq)) <= _summary_tol(wl.q, S)
    assert np.max(np.abs(host(kbar) - rk)) <= _summary_tol(wl.k, S)


def test_pooled_qk_video_size(bsa):
    """All 40 heads of the 21x30x52 video workload (S = 32760), the size the benchmark runs."""
    wl = make_config(2)
    say("pooled_qk video B1 H40 S32760 D128 bf16")
    qbar, kbar = bsa.api.pooled_qk(dev(wl.q, "bf16"), dev(wl.k, "bf16"))
    torch.cuda.synchronize()
    rq, rk = orr.pooled_summary(wl.q, wl.k, wl.Hq)
    assert np.max(np.abs(host(qbar) - rq)) <= _summary_tol(wl.q, wl.S)
    assert np.max(np.abs(host(kbar) - rk)) <= _summary_tol(wl.k, wl.S)


def _midpoint_delta(drift_row: np.ndarray, n_asking: int) -> float:
    """A threshold with exactly n_asking drifts above it, midway between two drifts."""
    d = np.sort(drift_row)[::-1]
    if n_asking == 0:
        return float(d[0] * 1.5 + 1.0)
    if n_asking == d.size:
        return float(d[-1] * 0.5)
    return float(0.5 * (d[n_asking - 1] + d[n_asking]))


@pytest.mark.parametrize("relative", [False, True])
@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("n_asking", [0, 3, 4, 6, 8, 9, 10])
def test_decide(bsa, relative, gate, n_asking):
    """Hm = 10 heads per batch entry: 3 asking (30%, gated to none), 4 (exactly 40%), 6, 8
    (exactly 80%), 9 (90%, gated to all), 10; two batch entries with the same counts."""
    rng = np.random.default_rng(100 + n_asking + 10 * relative)
    B, Hm, D = 2, 10, 128
    qbar, kbar = rng.standard_normal((B, Hm, D)), rng.standard_normal((B, Hm, D))
    # anchors at growing distances, so drifts are well separated
    scale = np.linspace(0.1, 2.0, Hm)[None, :, None] * rng.permutation(np.arange(1, Hm + 1))[None, :, None] / Hm
    aq = qbar + scale * rng.standard_normal((B, Hm, D))
    ak = kbar + scale * rng.standard_normal((B, Hm, D))
    f32 = lambda x: x.astype(np.float32)
    qbar, kbar, aq, ak = map(lambda x: f32(x).astype(np.float64), (qbar, kbar, aq, ak))
    ref_drift = orr.l1_drift(qbar, kbar, aq, ak, relative)
    # one threshold for the call: place it for batch entry 0, check entry 1 is equally robust
    delta = np.float32(_midpoint_delta(ref_drift[0], n_asking))
    gap = np.min(np.abs(ref_drift - float(delta)))
    assert gap > 1e-3 * max(1.0, float(delta)), "test inputs too close to the threshold"
    say(f"decide relative={relative} gate={gate} asking={n_asking} delta={float(delta):.4f}")
    t = lambda x: torch.from_numpy(f32(x)).cuda()
    drift, refresh = bsa.api.mask_reuse_decide(t(qbar), t(kbar), t(aq), t(ak), float(delta), relative, gate)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(drift), ref_drift, rtol=1e-5, atol=1e-6)
    want = orr.refresh_decision(ref_drift, float(delta), True, gate)
    assert refresh.cpu().numpy().astype(bool).tolist() == want.tolist()


def test_decide_first_call_and_zero_anchor(bsa):
    z = torch.zeros(1, 3, 4, device="cuda")
    drift, refresh = bsa.api.mask_reuse_decide(z, z, None, None, 0.5)
    assert refresh.cpu().tolist() == [[1, 1, 1]]
    cur = torch.tensor([[[0.0, 0, 0, 0], [0, 1.0, 0, 0], [0, 0, 0, 0]]], device="cuda")
    drift, refresh = bsa.api.mask_reuse_decide(cur, z, z, z, 0.5, relative=True, gate=False)
    d = drift.cpu().numpy()
    assert d[0, 0] == 0.0 and np.isinf(d[0, 1]) and refresh.cpu().tolist() == [[0, 1, 0]]


def test_update(bsa):
    rng = np.random.default_rng(7)
    B, Hm, Cq, Ck, D = 2, 6, 33, 31, 64
    say("mask_reuse_update B=2 Hm=6 Cq=33 Ck=31")
    refresh = (rng.random((B, Hm)) < 0.5).astype(np.uint8)
    new_keep = (rng.random((B, Hm, Cq, Ck)) < 0.3).astype(np.uint8)
    old_keep = (rng.random((B, Hm, Cq, Ck)) < 0.3).astype(np.uint8)
    new_cnt, old_cnt = rng.integers(0, Ck, (B, Hm, Cq)).astype(np.int32), rng.integers(0, Ck, (B, Hm, Cq)).astype(np.int32)
    new_idx = rng.integers(0, Ck, (B, Hm, Cq, Ck)).astype(np.int16)
    old_idx = rng.integers(0, Ck, (B, Hm, Cq, Ck)).astype(np.int16)
    qbar, kbar = rng.standard_normal((B, Hm, D)).astype(np.float32), rng.standard_normal((B, Hm, D)).astype(np.float32)
    aq, ak = rng.standard_normal((B, Hm, D)).astype(np.float32), rng.standard_normal((B, Hm, D)).astype(np.float32)
    c = lambda x: torch.from_numpy(x.copy()).cuda()
    new = bsa.BlockMask(c(new_keep), c(new_cnt), c(new_idx))
    cache = bsa.BlockMask(c(old_keep), c(old_cnt), c(old_idx))
    taq, tak = c(aq), c(ak)
    bsa.api.mask_reuse_update(c(refresh), c(qbar), c(kbar), new, cache, taq, tak)
    torch.cuda.synchronize()
    r = refresh.astype(bool)
    assert np.array_equal(cache.keep.cpu().numpy(), np.where(r[:, :, None, None], new_keep, old_keep))
    assert np.array_equal(cache.kv_count.cpu().numpy(), np.where(r[:, :, None], new_cnt, old_cnt))
    assert np.array_equal(cache.kv_idx.cpu().numpy(), np.where(r[:, :, None, None], new_idx, old_idx))
    assert np.array_equal(taq.cpu().numpy(), np.where(r[:, :, None], qbar, aq))
    assert np.array_equal(tak.cpu().numpy(), np.where(r[:, :, None], kbar, ak))
    # anchors only
    taq2, tak2 = c(aq), c(ak)
    bsa.api.mask_reuse_update(c(refresh), c(qbar), c(kbar), None, None, taq2, tak2)
    torch.cuda.synchronize()
    assert np.array_equal(taq2.cpu().numpy(), np.where(r[:, :, None], qbar, aq))


@pytest.mark.parametrize("pool", [False, True])
def test_scores_head_filter(bsa, pool):
    """Flagged heads get exactly the full scorer's rows; the other rows stay untouched."""
    wl = make_custom(404, B=1, Hq=4, Hkv=2, S=1100, D=128, dtype="bf16", block=128)
    q, k = dev(wl.q, "bf16"), dev(wl.k, "bf16")
    say(f"scores head filter pool={pool}")
    full = bsa.antidiagonal_block_scores(q, k, pool_gqa=pool)
    Hs = full.shape[1]
    heads = torch.tensor([[1, 0, 0, 1][:Hs]], dtype=torch.uint8, device="cuda")
    out = torch.full_like(full, -7.0)
    bsa.antidiagonal_block_scores(q, k, pool_gqa=pool, heads=heads, out=out)
    torch.cuda.synchronize()
    f, o = full.cpu().numpy(), out.cpu().numpy()
    for h in range(Hs):
        if heads[0, h]:
            assert np.array_equal(o[0, h], f[0, h])
        else:
            assert np.all(o[0, h] == -7.0)


def test_cache_steps_match_oracle(bsa):
    """Three steps of the device cache against the oracle cache on the same inputs: step
    t's queries and keys drift from step 0's by t * eps_h per head; the masks come from each
    side's own scoring and top-p of the refreshed heads."""
    base = make_custom(500, B=1, Hq=5, Hkv=5, S=1024, D=64, dtype="f32", block=128)
    rng = np.random.default_rng(501)
    dirs_q = rng.standard_normal((1, 5, 1, 64))
    dirs_q /= np.abs(dirs_q).sum(axis=-1, keepdims=True)  # unit L1 norm per head
    # per-step drift of each head from a step-0 anchor: 0, 0.7, 2.6, 15, 30 (delta = 2): step 1
    # asks for heads 2-4 (60%, per-head decisions), step 2 again for heads 2-4 against their
    # moved anchors while head 1 reaches 1.4 < 2 against its step-0 anchor
    eps = np.array([0.0, 0.7, 2.6, 15.0, 30.0])[None, :, None, None]
    delta = 2.0
    dc = bsa.api.HeadMaskCache(delta, gate=True)
    oc = orr.HeadMaskCache(delta, gate=True)
    scores_out = None
    for step in range(3):
        q = (base.q + step * eps * dirs_q).astype(np.float32)
        k = base.k
        say(f"cache step {step}")
        refresh = dc.should_refresh(dev(q, "f32"), dev(k, "f32"))
        o_refresh = oc.should_refresh(q, k, 5)
        torch.cuda.synchronize()
        margin = np.min(np.abs(oc.last_drift - delta)) if step > 0 else np.inf
        assert margin > 1e-3, "drift too close to delta for a robust comparison"
        assert refresh.cpu().numpy().astype(bool).tolist() == o_refresh.tolist()
        if scores_out is None:
            scores_out = torch.empty(1, 5, 8, 8, dtype=torch.float32, device="cuda")
        bsa.antidiagonal_block_scores(dev(q, "f32"), dev(k, "f32"), heads=refresh, out=scores_out)
        mask = dc.update(bsa.top_p_block_mask(scores_out, 0.9), refresh)
        o_mask = oc.update(np.zeros((1, 5, 8, 8), np.uint8) + step + 1, o_refresh)
        torch.cuda.synchronize()
        # which step built each head's cached mask: the oracle's marker; the device mask of
        # a head must equal the top-p mask computed at that step
        built = o_mask[0, :, 0, 0] - 1
        if step == 0:
            first = mask.keep.cpu().numpy().copy()
        for h in range(5):
            if built[h] == 0:
                assert np.array_equal(mask.keep.cpu().numpy()[0, h], first[0, h])


def test_path_with_cache(bsa):
    """The whole path with a mask cache: the first call equals the path without a cache; a
    second call on the same inputs reuses every mask and returns the same output; a call where
    one head's queries moved far rebuilds that head's mask only (other heads' rows equal
    the first call's)."""
    from synthetic.workloads import make_custom as mk
    wl = mk(610, B=1, Hq=5, Hkv=5, S=1024, D=128, dtype="bf16", block=128, mask="scored", probes=0)
    cfg = bsa.PathConfig.from_workload(wl)
    cfg.overlap = False
    path = bsa.SparseAttentionPath(cfg)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    say("path with cache")
    plain = path(q, k, v).out.float().cpu().numpy()
    cache = bsa.HeadMaskCache(delta=50.0, gate=False)
    first = path(q, k, v, cache=cache).out.float().cpu().numpy()
    assert np.array_equal(first, plain)
    keep0 = cache.mask.keep.cpu().numpy().copy()
    again = path(q, k, v, cache=cache).out.float().cpu().numpy()
    assert np.array_equal(again, first)
    assert float(cache.drift.max().item()) == 0.0
    q2 = wl.q.copy()
    q2[:, 3] = -q2[:, 3] + 3.0  # head 3 only: its mean moves by far more than delta
    out2 = path(dev(q2, "bf16"), k, v, cache=cache).out.float().cpu().numpy()
    d = cache.drift.cpu().numpy()[0]
    assert d[3] > 50.0 and np.all(np.delete(d, 3) == 0.0)
    keep2 = cache.mask.keep.cpu().numpy()
    assert np.array_equal(np.delete(keep2, 3, axis=1), np.delete(keep0, 3, axis=1))
    assert np.array_equal(np.delete(out2, 3, axis=1), np.delete(first, 3, axis=1))
