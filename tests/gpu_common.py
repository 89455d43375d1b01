"""Helpers shared by the GPU parity tests (host-side comparison only)."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import topp

# Tolerances: float32 inputs -> max-abs error; bfloat16 inputs -> relative L2 error per
# (batch, head) (the pages' workload statement fixes both bars).
F32_MAX_ABS = 1e-4
BF16_REL_L2 = 5e-3


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host float32 array (exactly representable in dtype) -> device tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


# Every mask comparison of the session: (what, rows with a fragile block, rows, bound).
FRAGILE: list = []

# Every output comparison of the session: (what, metric, error, bound).  The terminal summary
# (tests/conftest.py) prints the worst margins, so they are on record even under -q.
ERRORS: list = []


def check_output(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        ERRORS.append((what, "max-abs", err, F32_MAX_ABS))
        print(f"[err] {what}: max-abs {err:.3e}", flush=True)
        assert err <= F32_MAX_ABS, f"{what}: max-abs error {err:.3e} > {F32_MAX_ABS}"
    else:
        err = rel_l2(got, ref)
        ERRORS.append((what, "rel-L2", err, BF16_REL_L2))
        print(f"[err] {what}: rel-L2 {err:.3e}", flush=True)
        assert err <= BF16_REL_L2, f"{what}: rel-L2 error {err:.3e} > {BF16_REL_L2}"
    return err


def round_bf16(x) -> np.ndarray:
    """Round values to bfloat16 (nearest, ties to even), returned as float64: the rounding a
    kernel applies when it hands a float32 result to a bfloat16 product (test-side input
    preparation, not part of the oracle)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


ROUTE_TIE_REL = 1e-6  # float32 quotients of float32 values tie only within 2^-23 relative


def route_fragile_rows(err, k_counts, budget, eps_rel: float = ROUTE_TIE_REL) -> np.ndarray:
    """bool [..., rows]: rows whose error-aware route may differ between a float32 and a
    float64 evaluation of the ratios err / n_c.  Rounding cannot swap two quotients, only tie
    them (then the lower index goes first), so a route can change only when the last kept
    cluster sits in a run of near-equal float64 ratios that are not all exactly equal."""
    err = np.asarray(err, dtype=np.float64)
    n = np.asarray(k_counts, dtype=np.int64)
    nz = np.nonzero(n > 0)[0]
    out = np.zeros(err.shape[:-1], dtype=bool)
    for idx in np.ndindex(*err.shape[:-1]):
        ratio = err[idx][nz] / n[nz]
        order = np.lexsort((nz, -ratio))
        r = ratio[order]
        total, last = 0, len(order) - 1
        for i, j in enumerate(order):
            total += n[nz[j]]
            if total >= budget:
                last = i
                break
        lo = hi = last
        close = lambda a, b: abs(a - b) <= eps_rel * max(abs(a), abs(b))
        while lo > 0 and close(r[lo - 1], r[lo]):
            lo -= 1
        while hi + 1 < r.size and close(r[hi + 1], r[hi]):
            hi += 1
        out[idx] = bool(np.any(r[lo:hi + 1] != r[last]))
    return out


MAX_FRAGILE_ROW_FRACTION = 0.10  # rows with an excluded block, per mask head


def compare_masks(gpu_keep: np.ndarray, gpu_cnt: np.ndarray, gpu_idx: np.ndarray, oracle_scores: np.ndarray,
                  tau: float, what: str, eps_tie: float = 1e-6,
                  max_fragile: float = MAX_FRAGILE_ROW_FRACTION) -> dict:
    """Mask parity for one mask head ([rows, Ck] keep bits, counts, lists).

    * Every row's GPU list is exactly the ascending nonzero positions of its GPU keep bits.
    * Keep bits equal the oracle's top-p of its own scores on every block that is not fragile
      (decided within rounding of tau, or near-tied across the cut).
    * A row with a fragile block must still be a valid top-p set under the oracle's scores:
      its mass reaches tau of the row total within the fragility window, and dropping its
      smallest kept block falls short of it.
    * At most ``max_fragile`` of the rows hold a fragile block (the count is printed).

    ``eps_tie`` = 0 when both sides sort the very same score values (then only the prefix sums
    can round differently).
    """
    rows = oracle_scores.shape[0]
    n_frag_rows = 0
    for a in range(rows):
        got_list = np.nonzero(gpu_keep[a])[0]
        assert gpu_cnt[a] == got_list.size, f"{what}: row {a} count {gpu_cnt[a]} != {got_list.size} keep bits"
        assert np.array_equal(gpu_idx[a, : gpu_cnt[a]], got_list), f"{what}: row {a} list != its keep bits"
        want = topp.top_p_row(oracle_scores[a], tau)
        frag = topp.fragile_blocks(oracle_scores[a], tau, eps_tie=eps_tie)
        bad = (gpu_keep[a] != want) & ~frag
        assert not bad.any(), f"{what}: row {a} keep bits differ at blocks {np.nonzero(bad)[0][:8]}"
        if frag.any():
            n_frag_rows += 1
            s = np.asarray(oracle_scores[a], dtype=np.float64)
            kept = s[gpu_keep[a] != 0]
            target = tau * s.sum()
            assert kept.size >= 1 and kept.sum() >= target - 1e-5, f"{what}: row {a} kept mass short of tau"
            assert kept.sum() - kept.min() < target + 1e-5, f"{what}: row {a} keeps more blocks than needed"
    frac = n_frag_rows / max(rows, 1)
    print(f"[mask] {what}: {n_frag_rows} of {rows} rows hold a fragile block", flush=True)
    FRAGILE.append((what, n_frag_rows, rows, max_fragile))
    assert frac <= max_fragile, f"{what}: {n_frag_rows} of {rows} rows fragile"
    return dict(fragile_rows=n_frag_rows)
