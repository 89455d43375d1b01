"""Pins for the oracle's attention, probe and repair stages (CPU only).

The compensated attention is checked against a second, independent formulation of the
page (one collapsed term per skipped cluster, pure-Python loops), against PyTorch's
scaled_dot_product_attention in float64 (dense and token-masked), and against identities
the pages state (identical keys make compensation exact; the hard-drop residual equals
the omitted mass times the omitted-vs-sparse output gap).  The fit is checked against
hand-worked fixtures, the ridge optimality condition, weighted least squares from NumPy,
SVD-based principal directions and invariances.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import centroids as oc
from oracle import pipeline as op
from oracle import repair as orp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def sdpa64(q, k, v, scale, mask=None):
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)[0, 0].numpy()


def random_case(seed, Sq=40, Sk=56, D=6, Cq=5, Ck=7, p=0.4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Sq, D))
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    ql = rng.integers(0, Cq, size=Sq)
    kl = rng.integers(0, Ck, size=Sk)
    keep = (rng.uniform(size=(Cq, Ck)) < p).astype(np.uint8)
    return q, k, v, ql, kl, keep


# ---------------------------------------------------------------- attention


def test_compensation_golden():
    g = golden("compensation_tiny.json")
    q, v = np.array(g["q"]), np.array(g["values"])
    lab = np.array(g["labels"])
    keep = np.array(g["keep"])
    for keys, dense_key in (("keys_identical", "dense_identical"), ("keys_spread", "dense_spread")):
        k = np.array(g[keys])
        o, _ = oa.compensated_attention(q, k, v, np.array([0]), lab, keep, 1.0, True)
        assert abs(o[0, 0] - g["compensated"]) < 1e-14
        o, _ = oa.compensated_attention(q, k, v, np.array([0]), lab, keep, 1.0, False)
        assert abs(o[0, 0] - g["hard_drop"]) < 1e-14
        d = oa.dense_attention_rows(q, k, v, 1.0)
        assert abs(d[0, 0] - g[dense_key]) < 1e-14


def collapsed_form(q, k, v, ql, kl, keep, scale, compensate, given=None):
    """[SBC] SVG-EAR form, written per cluster with Python loops: kept clusters contribute
    every key; each skipped non-empty cluster contributes n_c * exp(q . kbar_c * scale)
    with value vbar_c.  ``given`` = (kbar, vbar, counts): the caller's centroid columns (a
    count of 0 contributes nothing)."""
    Sq, D = q.shape
    Ck = keep.shape[1]
    out = np.zeros((Sq, D))
    for i in range(Sq):
        terms = []  # (logit, weight multiplier, value)
        for c in range(Ck):
            idx = [j for j in range(k.shape[0]) if kl[j] == c]
            if not idx:
                continue
            if keep[ql[i], c]:
                for j in idx:
                    terms.append((float(q[i] @ k[j]) * scale, 1.0, v[j]))
            elif compensate and given is not None:
                if given[2][c] > 0:
                    terms.append((float(q[i] @ given[0][c]) * scale, float(given[2][c]), given[1][c]))
            elif compensate:
                kb = sum(k[j] for j in idx) / len(idx)
                vb = sum(v[j] for j in idx) / len(idx)
                terms.append((float(q[i] @ kb) * scale, float(len(idx)), vb))
        if not terms:
            continue
        m = max(t[0] for t in terms)
        num = sum(w * math.exp(s - m) * val for s, w, val in terms)
        den = sum(w * math.exp(s - m) for s, w, val in terms)
        out[i] = num / den
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("compensate", [True, False])
def test_extended_key_form_equals_collapsed_form(seed, compensate):
    q, k, v, ql, kl, keep = random_case(seed)
    o, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.4, compensate)
    assert np.allclose(o, collapsed_form(q, k, v, ql, kl, keep, 0.4, compensate), atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_caller_centroids(seed):
    """Centroid columns given by the caller: the extended-key form equals the per-cluster loop
    with those centroids and counts (a count of 0 removes the column), and giving the clusters'
    own means and sizes reproduces the default."""
    q, k, v, ql, kl, keep = random_case(seed)
    Ck, D = keep.shape[1], k.shape[1]
    rng = np.random.default_rng(100 + seed)
    kb, vb = rng.standard_normal((Ck, D)), rng.standard_normal((Ck, D))
    n = rng.integers(0, 9, Ck)
    n[0] = 0
    o, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.4, True, kbar=kb, vbar=vb, counts=n)
    want = collapsed_form(q, k, v, ql, kl, keep, 0.4, True, given=(kb, vb, n))
    assert np.allclose(o, want, atol=1e-13)
    kb0, vb0, n0 = oc.centroids(k, v, kl, Ck)
    o0, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.4, True, kbar=kb0, vbar=vb0, counts=n0)
    assert np.array_equal(o0, oa.compensated_attention(q, k, v, ql, kl, keep, 0.4, True)[0])


def test_all_kept_is_dense_sdpa():
    q, k, v, ql, kl, _ = random_case(10)
    keep = np.ones((5, 7), dtype=np.uint8)
    for comp in (True, False):
        o, lse = oa.compensated_attention(q, k, v, ql, kl, keep, 0.3, comp)
        assert np.allclose(o, sdpa64(q, k, v, 0.3), atol=1e-13)
        ref_lse = np.log(np.exp(0.3 * q @ k.T).sum(axis=1))
        assert np.allclose(lse, ref_lse, atol=1e-12)


def test_identical_keys_make_compensation_exact():
    rng = np.random.default_rng(11)
    Sk, D, Ck = 60, 5, 6
    kl = rng.integers(0, Ck, size=Sk)
    cent = rng.standard_normal((Ck, D))
    k = cent[kl]
    v = rng.standard_normal((Sk, D)) * 3
    q = rng.standard_normal((30, D))
    ql = rng.integers(0, 4, size=30)
    for trial in range(5):
        keep = (rng.uniform(size=(4, Ck)) < 0.3).astype(np.uint8)
        o, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.6, True)
        assert np.allclose(o, sdpa64(q, k, v, 0.6), atol=1e-13)


def test_hard_drop_is_token_masked_sdpa():
    q, k, v, ql, kl, keep = random_case(12)
    keep[:, 0] = 1  # every row keeps something
    o, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.5, False)
    tok = np.where(keep[ql][:, kl] != 0, 0.0, -np.inf)
    assert np.allclose(o, sdpa64(q, k, v, 0.5, tok), atol=1e-13)


def test_hard_drop_residual_identity():
    # [SPR]: under renormalized hard drop, O_dense - O_sparse equals the omitted mass times
    # (omitted-support output - sparse output).
    q, k, v, ql, kl, keep = random_case(13)
    keep[:, 0] = 1
    keep[:, 1] = 0
    o_s, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.5, False)
    kept_tok = keep[ql][:, kl] != 0
    o_d = sdpa64(q, k, v, 0.5)
    o_omit = sdpa64(q, k, v, 0.5, np.where(kept_tok, -np.inf, 0.0))
    p = np.exp(0.5 * q @ k.T)
    alpha = (p * ~kept_tok).sum(axis=1) / p.sum(axis=1)
    assert np.allclose(o_d - o_s, alpha[:, None] * (o_omit - o_s), atol=1e-13)


def test_outputs_are_convex_combinations():
    q, k, _, ql, kl, keep = random_case(14)
    Sk = k.shape[0]
    o, _ = oa.compensated_attention(q, k, np.eye(Sk), ql, kl, keep, 0.5, True)
    assert np.all(o >= -1e-15)
    assert np.allclose(o.sum(axis=1), 1.0, atol=1e-13)
    const = np.tile(np.array([[2.0, -1.0, 0.5]]), (Sk, 1))
    o, _ = oa.compensated_attention(q, k, const, ql, kl, keep, 0.5, True)
    assert np.allclose(o, const[:1], atol=1e-13)


def test_empty_cluster_and_empty_row():
    q, k, v, ql, kl, keep = random_case(15, Ck=7)
    kl = np.where(kl == 3, 4, kl)  # cluster 3 empty
    o1, _ = oa.compensated_attention(q, k, v, ql, kl, keep, 0.5, True)
    keep2 = keep.copy()
    keep2[:, 3] = 1 - keep2[:, 3]  # an empty cluster's bit changes nothing
    o2, _ = oa.compensated_attention(q, k, v, ql, kl, keep2, 0.5, True)
    assert np.allclose(o1, o2, atol=1e-15)
    keep3 = keep.copy()
    keep3[ql[0]] = 0  # a row with nothing kept: hard drop gives 0 and lse -inf
    o3, lse3 = oa.compensated_attention(q, k, v, ql, kl, keep3, 0.5, False)
    assert np.all(o3[ql == ql[0]] == 0) and np.all(np.isneginf(lse3[ql == ql[0]]))


def test_row_subset_and_dense_rows():
    q, k, v, ql, kl, keep = random_case(16)
    o, lse = oa.compensated_attention(q, k, v, ql, kl, keep, 0.5, True)
    rows = np.array([5, 0, 17])
    o2, lse2 = oa.compensated_attention(q, k, v, ql, kl, keep, 0.5, True, rows=rows, chunk=2)
    assert np.allclose(o2, o[rows], atol=1e-15) and np.allclose(lse2, lse[rows])
    assert np.allclose(oa.dense_attention_rows(q[rows], k, v, 0.5), sdpa64(q, k, v, 0.5)[rows], atol=1e-13)


# ---------------------------------------------------------------- probes


def test_probe_selection_golden():
    g = golden("probes_tiny.json")
    for case in g["cases"]:
        idx, w = orp.select_probe_rows(np.array(g["labels"]), g["C"], case["M"])
        assert idx.tolist() == case["probe_idx"]
        assert np.allclose(w, case["weights"], atol=1e-15)


def test_probe_selection_properties():
    rng = np.random.default_rng(20)
    labels = rng.integers(0, 9, size=400)
    for M in (1, 5, 9, 30, 64, 400):
        idx, w = orp.select_probe_rows(labels, 9, M)
        assert len(set(idx.tolist())) == M and abs(w.sum() - 1) < 1e-14 and np.all(w > 0)
        per = np.bincount(labels[idx], minlength=9)
        if M >= 9 and M <= 9 * np.bincount(labels).min():
            assert per.max() - per.min() <= 1
    # one probe per cluster: the middle-out (middle) member
    idx, _ = orp.select_probe_rows(labels, 9, 9)
    for a in range(9):
        mem = np.nonzero(labels == a)[0]
        assert idx[a] == mem[len(mem) // 2]
    assert orp.middle_out(6) == [3, 2, 4, 1, 5, 0]


# ---------------------------------------------------------------- ridge fit


def test_ridge_golden_1d():
    g = golden("ridge_1d.json")
    fit = orp.ridge_fit(np.array(g["o_sparse"]), np.array(g["o_dense"]), np.array(g["weights"]), g["lam"], g["rank"])
    for key in ("mu", "sigma", "rbar", "W", "A", "c"):
        assert np.allclose(fit[key], g[key], atol=1e-14), key
    corr = orp.apply_correction(np.array(g["o_sparse"]), fit["A"], fit["c"]) - np.array(g["o_sparse"])
    assert np.allclose(corr, g["corrections"], atol=1e-14)


def fit_case(seed, M=64, D=16, scale_res=0.1):
    rng = np.random.default_rng(seed)
    xs = rng.standard_normal((M, D)) * rng.uniform(0.5, 2, size=D) + rng.standard_normal(D)
    xd = xs + scale_res * (xs @ rng.standard_normal((D, D)) * 0.2 + rng.standard_normal((M, D)))
    w = rng.uniform(0.5, 3, size=M)
    return xs, xd, w


def test_ridge_optimality_condition():
    xs, xd, w = fit_case(21)
    fit = orp.ridge_fit(xs, xd, w, 0.1, 16)
    wn = w / w.sum()
    X, Rc, W = fit["X"], fit["Rc"], fit["W"]
    lhs = X.T @ (wn[:, None] * (Rc - X @ W))
    assert np.allclose(lhs, 0.1 * W, atol=1e-13)
    assert np.allclose(wn @ X, 0, atol=1e-13) and np.allclose(wn @ X ** 2, 1, atol=1e-13)


def test_ridge_small_lambda_full_rank_is_weighted_least_squares():
    xs, xd, w = fit_case(22, M=80, D=6)
    fit = orp.ridge_fit(xs, xd, w, 1e-12, 6)
    wn = w / w.sum()
    design = np.concatenate([xs, np.ones((80, 1))], axis=1) * np.sqrt(wn)[:, None]
    coef, *_ = np.linalg.lstsq(design, (xd - xs) * np.sqrt(wn)[:, None], rcond=None)
    assert np.allclose(fit["A"], coef[:6], atol=1e-8)
    assert np.allclose(fit["c"], coef[6], atol=1e-8)


def test_small_lambda_full_rank_interpolates_probes():
    xs, xd, w = fit_case(23, M=10, D=16)
    fit = orp.ridge_fit(xs, xd, w, 1e-10, 16)
    rep = orp.apply_correction(xs, fit["A"], fit["c"])
    assert np.allclose(rep, xd, atol=1e-6)


def test_projector_matches_svd_directions():
    xs, xd, w = fit_case(24, M=64, D=32)
    fit = orp.ridge_fit(xs, xd, w, 0.1, 16)
    P = fit["P"]
    assert np.allclose(P @ P, P, atol=1e-12) and abs(np.trace(P) - 16) < 1e-10
    wn = w / w.sum()
    _, _, vt = np.linalg.svd(np.sqrt(wn)[:, None] * fit["Rc"], full_matrices=False)
    assert np.allclose(P, vt[:16].T @ vt[:16], atol=1e-8)
    assert np.allclose(orp.correction(xs, fit), xs @ fit["A"] + fit["c"], atol=1e-12)


def test_zero_residual_gives_zero_correction_and_rank_drop():
    xs, _, w = fit_case(25)
    fit = orp.ridge_fit(xs, xs, w, 0.1, 16)
    assert fit["r_eff"] == 0 and np.all(fit["A"] == 0) and np.all(fit["c"] == 0)
    # residuals in a 3-dimensional subspace: only 3 directions are kept
    rng = np.random.default_rng(26)
    basis = rng.standard_normal((3, 16))
    xd = xs + rng.standard_normal((64, 3)) @ basis
    fit = orp.ridge_fit(xs, xd, w, 0.1, 16)
    assert fit["r_eff"] == 3


def test_integer_weights_equal_duplicated_rows_and_order_irrelevant():
    xs, xd, _ = fit_case(27, M=20, D=8)
    reps = np.arange(20) % 3 + 1
    fit_w = orp.ridge_fit(xs, xd, reps.astype(float), 0.1, 4)
    fit_d = orp.ridge_fit(np.repeat(xs, reps, axis=0), np.repeat(xd, reps, axis=0), np.ones(reps.sum()), 0.1, 4)
    assert np.allclose(fit_w["A"], fit_d["A"], atol=1e-12) and np.allclose(fit_w["c"], fit_d["c"], atol=1e-12)
    p = np.random.default_rng(0).permutation(20)
    fit_p = orp.ridge_fit(xs[p], xd[p], reps[p].astype(float), 0.1, 4)
    assert np.allclose(fit_w["A"], fit_p["A"], atol=1e-12)


def test_standardization_makes_fit_invariant_to_feature_affine_maps():
    xs, xd, w = fit_case(28, M=40, D=8)
    fit = orp.ridge_fit(xs, xd, w, 0.1, 8)
    s = np.random.default_rng(1).uniform(0.2, 5, size=8)
    b = np.random.default_rng(2).standard_normal(8)
    xs2 = xs * s + b
    xd2 = xd - xs + xs2  # same residuals
    fit2 = orp.ridge_fit(xs2, xd2, w, 0.1, 8)
    assert np.allclose(orp.correction(xs, fit), orp.correction(xs2, fit2), atol=1e-12)


def test_repaired_probe_rows_match_dense_up_to_fit_residual():
    xs, xd, w = fit_case(29)
    fit = orp.ridge_fit(xs, xd, w, 0.1, 16)
    rep = orp.apply_correction(xs, fit["A"], fit["c"])
    assert np.allclose(rep - xd, fit["X"] @ fit["W"] @ fit["P"] - fit["Rc"], atol=1e-12)


# ---------------------------------------------------------------- composed path


class _WL:
    pass


def test_pipeline_small_case_runs_and_repairs_probes():
    rng = np.random.default_rng(30)
    wl = _WL()
    wl.B, wl.Hq, wl.Hkv, S, D = 1, 2, 1, 256, 16
    wl.q = rng.standard_normal((1, 2, S, D))
    wl.k = rng.standard_normal((1, 1, S, D))
    wl.v = rng.standard_normal((1, 1, S, D))
    wl.labels = (np.arange(S) // 32).astype(np.int32)
    wl.C, wl.scale = 8, 0.25
    wl.mask_mode, wl.block, wl.stride, wl.score_scale = "scored", 32, 8, 0.25
    wl.tau = np.array([0.8], dtype=np.float32)
    wl.pool_gqa, wl.compensate, wl.probes, wl.lam, wl.rank = True, True, 16, 0.1, 4
    wl.mask = None
    res = op.run_head(wl, 0, 1)
    assert res["keep"].shape == (8, 8) and res["keep"].sum(axis=1).min() >= 1
    rep_p = res["out"][res["probe_idx"]]
    fit = res["fit"]
    assert np.allclose(rep_p - res["o_dense_p"], fit["X"] @ fit["W"] @ fit["P"] - fit["Rc"], atol=1e-12)
    assert np.allclose(res["o_dense_p"], sdpa64(wl.q[0, 1][res["probe_idx"]], wl.k[0, 0], wl.v[0, 0], 0.25), atol=1e-13)
