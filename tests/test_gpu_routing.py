"""GPU parity for error-aware routing: the query-centroid probes, the per-block compensation
errors and the routes, each against the oracle on the same seeded inputs (ragged clusters,
an empty cluster, more than one 128-row tile of probes, grouped-query heads)."""

import numpy as np
import pytest
import torch

from oracle import routing as ort
from synthetic import make_custom

from gpu_common import dev, host, round_bf16, route_fragile_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _sizes(seed, S, lo, hi, empty=(3,)):
    """Ragged cluster sizes summing to S, with empty clusters at the given indices."""
    rng = np.random.default_rng(seed)
    sizes, left = [], S
    while left > 0:
        if len(sizes) in empty:
            sizes.append(0)
            continue
        n = int(min(left, rng.integers(lo, hi)))
        sizes.append(n)
        left -= n
    return sizes


def _bf16_ulps(a, b):
    """Distance in bfloat16 steps between arrays of bfloat16 values (same sign assumed near 0)."""
    ia = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
    ib = torch.from_numpy(b.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


@pytest.mark.parametrize("dtype,D,S,Hq", [("bf16", 128, 1700, 3), ("bf16", 64, 2300, 2), ("f32", 128, 1300, 2)])
def test_query_centroids(bsa, dtype, D, S, Hq):
    say(f"query centroids {dtype} D={D} S={S}")
    wl = make_custom(21, B=2, Hq=Hq, Hkv=Hq, S=S, D=D, dtype=dtype, cluster_sizes=_sizes(5, S, 1, 160))
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    got = host(bsa.query_centroids(dev(wl.q, dtype), lay))
    want = ort.query_centroids(wl.q, wl.labels, wl.C)  # float64 means
    assert np.all(got[:, :, 3] == 0.0)  # the empty cluster
    if dtype == "bf16":
        # The kernel returns its float32 mean rounded to bfloat16: within one bfloat16 step of
        # the float64 mean's rounding (float32 sums in another order may round either way).
        ulps = _bf16_ulps(got, round_bf16(want))
        assert ulps.max() <= 1 and np.mean(ulps) < 0.01, (ulps.max(), np.mean(ulps))
    else:
        assert np.allclose(got, want, rtol=1e-5, atol=1e-6)


CASES = [  # seed, B, Hq, Hkv, S, D, cluster sizes (lo, hi)
    (31, 1, 2, 1, 1500, 128, (1, 200)),
    (32, 2, 2, 2, 2300, 64, (1, 160)),
    (33, 1, 1, 1, 4100, 128, (5, 36)),  # about 200 probes: two 128-row tiles
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,D,sizes", CASES)
def test_block_error(bsa, seed, B, Hq, Hkv, S, D, sizes):
    say(f"block error seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    wl = make_custom(seed, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", cluster_sizes=_sizes(seed, S, *sizes))
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    kv = bsa.kv_pack(dev(wl.k, "bf16"), dev(wl.v, "bf16"), lay)
    # The probes are an input of the error pass: the float64 means rounded to bfloat16, the
    # element type the kernel takes, hand both sides identical probe rows.
    qbar = round_bf16(ort.query_centroids(wl.q, wl.labels, wl.C))
    err = host(bsa.block_error(dev(qbar, "bf16"), kv, wl.scale))
    want = ort.block_compensation_error(qbar, wl.k, wl.v, wl.labels, wl.C, wl.scale)
    assert np.all(err[..., 3] == 0.0)  # the empty cluster
    # Relative to the entry and to its row's largest error, plus a floor for float32 rounding:
    # the error is a difference of sums whose terms are of the size of V (errors that vanish,
    # such as those of the zero probe of an empty query cluster, come out at ~1e-6 |V|).
    row_max = want.max(axis=-1, keepdims=True)
    bound = 1e-2 * want + 2e-3 * row_max + 1e-5 * np.abs(wl.v).max()
    excess = np.abs(err - want) - bound
    print(f"[err] block error: max |gpu - oracle| = {np.max(np.abs(err - want)):.3e} "
          f"(largest error {want.max():.3e}), worst excess over the bound {excess.max():.3e}", flush=True)
    assert excess.max() <= 0.0


@pytest.mark.parametrize("Ck,rows,budget", [(40, 64, 0), (40, 64, 1), (300, 50, 2000), (1024, 9, 20000),
                                            (7, 5, 10 ** 9)])
def test_error_route_bit_exact(bsa, Ck, rows, budget):
    """Seeded errors with many exact ties and quotient near-ties, cluster sizes with empty
    clusters.  The kernel orders by float32 quotients, the oracle by float64 ones; rounding
    can only tie near-equal quotients (then the lower index goes first), so every row whose
    cut is not inside a near-tied run of float64 ratios must match bit for bit, and the others
    must still be valid routes (budget reached, nothing ranked clearly below a dropped
    cluster kept)."""
    say(f"route Ck={Ck} rows={rows} budget={budget}")
    rng = np.random.default_rng(Ck + rows)
    n = rng.integers(0, 90, Ck)
    n[rng.random(Ck) < 0.1] = 0
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    err = (rng.integers(0, 40, (1, 1, rows, Ck)) / 8.0).astype(np.float32)
    err[..., ::5] *= np.float32(3.0)  # quotients that tie only after rounding
    class _L:  # the route reads only the key offsets (one layout for every row)
        offsets = torch.from_numpy(off).cuda()
        n_layouts = 1
    m = bsa.error_route(torch.from_numpy(err).cuda(), _L, budget)
    want = ort.error_aware_route(err, n, budget)
    fragile = route_fragile_rows(err, n, budget)[0, 0]
    keep = m.keep.cpu().numpy()
    cnt = m.kv_count.cpu().numpy()
    idx = m.kv_idx.cpu().numpy()
    ratio = err[0, 0].astype(np.float64) / np.maximum(n, 1)
    for r in range(rows):
        got = keep[0, 0, r]
        lst = np.nonzero(got)[0]
        assert cnt[0, 0, r] == lst.size and np.array_equal(idx[0, 0, r, :lst.size], lst), r
        if not fragile[r]:
            assert np.array_equal(got, want[0, 0, r]), r
            continue
        kr = got.astype(bool)
        assert lst.size >= 1 and not np.any(kr & (n == 0))
        assert n[kr].sum() >= budget or np.all(kr == (n > 0))
        dropped = ~kr & (n > 0)
        if dropped.any():
            assert ratio[r][kr].min() >= ratio[r][dropped].max() * (1 - 1e-6), r
    print(f"[err] route rows with a float32 near-tie at the cut: {int(fragile.sum())} of {rows}", flush=True)
    assert fragile.sum() <= max(2, rows // 10)


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,D,sizes", CASES[:2])
def test_routes_end_to_end(bsa, seed, B, Hq, Hkv, S, D, sizes):
    """Probes, errors and routes on the GPU.  Routes are compared with the oracle's where
    they are unique: every GPU route reaches the budget (or keeps every non-empty cluster) and
    most rows equal the oracle's; where a row differs, the blocks it swaps have oracle ratios
    within 5% of each other (near-ties) or errors at the float32 rounding floor."""
    say(f"routes end to end seed={seed}")
    wl = make_custom(seed, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", cluster_sizes=_sizes(seed, S, *sizes))
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    kv = bsa.kv_pack(dev(wl.k, "bf16"), dev(wl.v, "bf16"), lay)
    budget = int(0.25 * S)
    qbar = bsa.query_centroids(dev(wl.q, "bf16"), lay)
    err = bsa.block_error(qbar, kv, wl.scale)
    m = bsa.error_route(err, lay, budget)
    keep = m.keep.cpu().numpy().astype(bool)
    n = np.bincount(wl.labels, minlength=wl.C)
    oq = ort.query_centroids(wl.q, wl.labels, wl.C)  # float64 probes (the kernel's are bfloat16)
    oerr = ort.block_compensation_error(oq, wl.k, wl.v, wl.labels, wl.C, wl.scale)
    want = ort.error_aware_route(oerr, n, budget).astype(bool)
    same = 0
    for idx in np.ndindex(*keep.shape[:-1]):
        kr, wr = keep[idx], want[idx]
        assert not np.any(kr & (n == 0))
        tot = n[kr].sum()
        assert tot >= budget or np.all(kr == (n > 0))
        if np.array_equal(kr, wr):
            same += 1
            continue
        ratio = oerr[idx] / np.maximum(n, 1)
        lost, gained = ratio[wr & ~kr], ratio[kr & ~wr]
        if lost.size and gained.size:  # near-ties, or errors at the float32 rounding floor
            assert gained.min() >= 0.95 * lost.max() - 1e-5 * np.abs(wl.v).max(), (gained.min(), lost.max())
    rows = int(np.prod(keep.shape[:-1]))
    print(f"[err] routes equal to the oracle's: {same} of {rows}", flush=True)
    assert same >= 0.9 * rows


def test_block_error_video_sampled(bsa):
    """The video workload at full size (B 1, H 40, S 32760, D 128, 256 clusters) in the launch
    configuration the benchmark times; the oracle checks sampled probe rows one by one (its
    own probes; the GPU's are within one bfloat16 step of them), the ragged last cluster
    included, and the routes of those rows are checked for validity."""
    from synthetic import make_config

    say("routing video generate")
    wl = make_config(2)
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    k, v = dev(wl.k, "bf16"), dev(wl.v, "bf16")
    kv = bsa.kv_pack(k, v, lay)
    say("routing video gpu")
    qbar = bsa.query_centroids(dev(wl.q, "bf16"), lay)
    err = host(bsa.block_error(qbar, kv, wl.scale))
    budget = int(0.2 * wl.S)
    keep = bsa.error_route(torch.from_numpy(err.astype(np.float32)).cuda(), lay, budget).keep.cpu().numpy().astype(bool)
    n = np.bincount(wl.labels, minlength=wl.C)
    vmax = np.abs(wl.v).max()
    for h in (0, 17, 39):
        oq = ort.query_centroids(wl.q[:, h:h + 1], wl.labels, wl.C)  # float64 probes
        gq = host(qbar[:, h:h + 1])
        assert _bf16_ulps(gq, round_bf16(oq)).max() <= 1
        for a in (0, 101, wl.C - 1):
            say(f"routing video h{h} a{a}")
            want = ort.block_compensation_error(oq[:, :, a:a + 1], wl.k[:, h:h + 1], wl.v[:, h:h + 1], wl.labels, wl.C,
                                                wl.scale)[0, 0, 0]
            got = err[0, h, a]
            bound = 1e-2 * want + 2e-3 * want.max() + 1e-5 * vmax
            # the GPU's probe is the float64 mean rounded to bfloat16 (within one step)
            assert np.all(np.abs(got - want) <= 2 * bound), float(np.max(np.abs(got - want) - 2 * bound))
            kr = keep[0, h, a]
            assert n[kr].sum() >= budget and not np.any(kr & (n == 0))


def test_path_routed(bsa):
    """The whole path with error-aware routes in place of scores and top-p (compensated, no
    probes): its mask equals the stage-by-stage routes, and the rows of every query cluster
    whose route equals the oracle's match the oracle's compensated attention on that route."""
    from oracle import attention as oatt
    from gpu_common import check_output

    S, density = 1800, 0.3
    say("routed path")
    wl = make_custom(41, B=1, Hq=2, Hkv=1, S=S, D=128, dtype="bf16", cluster_sizes=_sizes(41, S, 20, 160))
    cfg = bsa.PathConfig.from_workload(wl)
    cfg.mask_mode, cfg.route_density = "routed", density
    path = bsa.SparseAttentionPath(cfg)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    res = path(q, k, v)
    torch.cuda.synchronize()
    budget = int(round(density * S))
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    err = bsa.block_error(bsa.query_centroids(q, lay), bsa.kv_pack(k, v, lay), wl.scale)
    keep = res.mask.keep.cpu().numpy()
    assert np.array_equal(keep, bsa.error_route(err, lay, budget).keep.cpu().numpy())
    n = np.bincount(wl.labels, minlength=wl.C)
    oq = ort.query_centroids(wl.q, wl.labels, wl.C)
    okeep = ort.error_aware_route(ort.block_compensation_error(oq, wl.k, wl.v, wl.labels, wl.C, wl.scale), n, budget)
    out = host(res.out)
    checked = 0
    for h in range(2):
        same = np.all(keep[0, h] == okeep[0, h], axis=1)
        rows = np.nonzero(same[wl.labels])[0]
        ref, _ = oatt.compensated_attention(wl.q[0, h], wl.k[0, 0], wl.v[0, 0], wl.labels, wl.labels, okeep[0, h],
                                            wl.scale, True, rows=rows)
        check_output(out[0, h][rows], ref, "bf16", f"routed path h{h}")
        checked += rows.size
    assert checked >= 0.8 * 2 * S
