"""Full-size parity of the partitioned (SparsePR) call on the video workload, in the launch
configuration the benchmark times: all 40 heads, 256 key and 256 query groups per head,
error-aware routes at 22% executed-pair density with the 64 probe rows' share reserved, hard
drop, the fit and the corrected attention ("Partition the Support, Reconstruct the Residual").

The oracle checks sampled heads given the path's own labels (whose validity against the
oracle's features is checked here too, and in test_gpu_partition): the block errors of the
path's router probes match the oracle's within the error pass's tolerance, the routes equal
the oracle's routes on those errors outside near-tied rows, the probes follow the selection
rule on the path's query groups, and sampled output rows -- the probe rows among them -- match
the oracle's hard-drop attention corrected by the oracle's fit of its own probe rows, on the
path's mask.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import partition as op
from oracle import repair as orep
from oracle import routing as ort
from synthetic import make_config

from gpu_common import check_output, dev, host, route_fragile_rows, say
from test_gpu_partition import check_nearest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def test_partitioned_video_sampled(bsa):
    say("partitioned video generate")
    wl = make_config(2)
    cfg = bsa.PathConfig.from_workload(dataclasses.replace(wl, compensate=False, probes=64, lam=0.1, rank=16))
    cfg.mask_mode, cfg.route_density = "partitioned", 0.22
    path = bsa.SparseAttentionPath(cfg)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    say("partitioned video gpu path")
    res = path(q, k, v)
    _, _, kc, qc = bsa.response_partition(q, k, wl.C, wl.C, wl.scale, return_centres=True)
    qbar_t = bsa.query_centroids(q, res.extras["q_layout"])
    err = host(bsa.block_error(qbar_t, bsa.kv_pack(k, v, res.layout), wl.scale))  # the path's router errors
    qbar = host(qbar_t)
    torch.cuda.synchronize()
    S, C, M = wl.S, wl.C, cfg.probes
    klab = res.extras["k_labels"].cpu().numpy().reshape(wl.Hkv, S)
    qlab = res.extras["q_labels"].cpu().numpy().reshape(wl.Hkv, S)
    kc, qc = kc.cpu().numpy().reshape(wl.Hkv, C, 64), qc.cpu().numpy().reshape(wl.Hkv, C, 64)
    keep = res.mask.keep.cpu().numpy()
    pidx, pw = res.extras["probe_idx"].cpu().numpy(), res.extras["probe_w"].cpu().numpy()
    budget = res.extras["budget"]
    assert budget == int(round(0.22 * S)) - M
    out = host(res.out)
    n_pairs = 0.0
    for h in range(wl.Hq):
        nq, nk = np.bincount(qlab[h], minlength=C), np.bincount(klab[h], minlength=C)
        n_pairs += float((keep[0, h] * nk[None, :]).sum(axis=1) @ nq)
    density = (n_pairs + wl.Hq * M * S) / (wl.Hq * float(S) ** 2)
    say(f"partitioned video executed-pair density {density:.4f}")
    assert abs(density - 0.22) < 0.01
    rng = np.random.default_rng(5)
    for h in (3, 29):
        say(f"partitioned video head {h}: partition")
        qh, kh, vh = wl.q[0, h], wl.k[0, h], wl.v[0, h]
        # the partition: labels are nearest centres (within rounding) in the oracle's features
        kf = op.key_features(kh, op.sampled_queries(qh[None]), wl.scale)
        check_nearest(kf, kc[h, :, :op.RK].astype(np.float64), klab[h], f"head {h} keys")
        qf = op.query_coordinates(qh[None], kh, klab[h], C, wl.scale)
        check_nearest(qf, qc[h, :, :qf.shape[1]].astype(np.float64), qlab[h], f"head {h} queries")
        say(f"partitioned video head {h}: block errors and routes")
        want = ort.block_compensation_error(qbar[:, h:h + 1], wl.k[:, h:h + 1], wl.v[:, h:h + 1], klab[h], C,
                                            wl.scale)
        bound = 1e-2 * want + 2e-3 * want.max(axis=-1, keepdims=True) + 1e-5 * np.abs(wl.v).max()
        assert np.all(np.abs(err[:, h:h + 1] - want) <= bound)
        e32 = err[:, h:h + 1].astype(np.float32)
        n = np.bincount(klab[h], minlength=C)
        same = np.all(keep[0, h] == ort.error_aware_route(e32, n, budget)[0, 0], axis=1)
        fragile = route_fragile_rows(e32, n, budget)[0, 0]
        assert np.all(same | fragile), f"head {h}: {np.sum(~same & ~fragile)} routes differ outside near ties"
        say(f"partitioned video head {h}: probes and rows")
        ri, rw = orep.select_probe_rows(qlab[h], C, M)
        assert np.array_equal(pidx[h], ri)
        np.testing.assert_allclose(pw[h], rw, rtol=2e-6)
        rows = np.unique(np.concatenate([rng.choice(S, size=320, replace=False), ri]))
        o_sparse, _ = oatt.compensated_attention(qh, kh, vh, qlab[h], klab[h], keep[0, h], wl.scale, False, rows=rows)
        od = oatt.dense_attention_rows(qh[ri], kh, vh, wl.scale)
        at = np.searchsorted(rows, ri)
        fit = orep.ridge_fit(o_sparse[at], od, rw, cfg.lam, cfg.rank)
        ref = orep.apply_correction(o_sparse, fit["A"], fit["c"])
        check_output(out[0, h][rows], ref, "bf16", f"partitioned video h{h}")
