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


def check_output(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        print(f"[err] {what}: max-abs {err:.3e}", flush=True)
        assert err <= F32_MAX_ABS, f"{what}: max-abs error {err:.3e} > {F32_MAX_ABS}"
    else:
        err = rel_l2(got, ref)
        print(f"[err] {what}: rel-L2 {err:.3e}", flush=True)
        assert err <= BF16_REL_L2, f"{what}: rel-L2 error {err:.3e} > {BF16_REL_L2}"
    return err


def compare_masks(gpu_keep: np.ndarray, gpu_cnt: np.ndarray, gpu_idx: np.ndarray, oracle_scores: np.ndarray,
                  tau: float, what: str) -> dict:
    """Keep bits must equal the oracle's top-p of its own scores except on fragile blocks
    (decided within rounding of tau, or near-tied across the cut); the kept-block list of
    every row without a fragile block must equal the oracle's exactly."""
    rows = oracle_scores.shape[0]
    n_frag_rows = 0
    for a in range(rows):
        want = topp.top_p_row(oracle_scores[a], tau)
        frag = topp.fragile_blocks(oracle_scores[a], tau)
        bad = (gpu_keep[a] != want) & ~frag
        assert not bad.any(), f"{what}: row {a} keep bits differ at blocks {np.nonzero(bad)[0][:8]}"
        if frag.any():
            n_frag_rows += 1
            continue
        want_list = np.nonzero(want)[0]
        assert gpu_cnt[a] == want_list.size, f"{what}: row {a} kept count {gpu_cnt[a]} != {want_list.size}"
        assert np.array_equal(gpu_idx[a, : gpu_cnt[a]], want_list), f"{what}: row {a} kept list differs"
    return dict(fragile_rows=n_frag_rows)
