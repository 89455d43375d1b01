"""The whole path as one call: layout -> centroids -> scores -> top-p -> (probe rows ->
fit) -> sparse attention with the correction in its epilogue.

Order of stages: "Dynamic block masks and head-wise mask reuse", section "Recipe" (scores,
top-p mask, labels, compensated attention) and "Sparse-block compensation", section
"Recipe: STA with both repairs" (compensated attention, probe selection, dense probe rows,
residual correction).  The probes' block-sparse rows are computed by the probe pass itself
(the same rule as the attention, "Partition the Support, Reconstruct the Residual": a few
exact probe rows against their sparse counterparts), so the fit is known before the
attention runs and every row is corrected before its single rounding.  Every stage is one
or a few kernel launches on the current stream; nothing is computed on the host except the
probe selection, which depends only on the labels and is done once.

Streams: the K/V packing depends only on the inputs and the layout, so with
``PathConfig.overlap`` it runs on a second stream (default priority) while the scores and the
top-p masks run on the caller's stream, and the probe rows and the attention wait for both.
The default runs it on the caller's stream before the scores: both kernels fill the chip, so
side by side each slows down by about what the other takes, and the call is no faster.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np
import torch

from . import _lib, api


@dataclass
class PathConfig:
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    labels: np.ndarray  # int32 [S] (host); unused by "partitioned" (its labels come from the call)
    C: int
    scale: float
    # "given", "scored", "routed" (error-aware routes under route_density) or "partitioned"
    # (response-coupled partitions per (batch, K/V head), then error-aware routes)
    mask_mode: str
    keep: Optional[np.ndarray] = None  # given mode: uint8 [B or 1, Hm, C, C]
    block: int = 128
    stride: int = 16
    score_scale: Optional[float] = None
    tau: Optional[np.ndarray] = None  # scored mode: [Hs]
    pool_gqa: bool = False
    compensate: bool = True
    probes: int = 0
    lam: float = 0.1
    rank: int = 16
    overlap: bool = False  # the pack on a second stream, beside scores and top-p (no faster)
    route_density: float = 0.2  # routed modes: executed-pair density (probe rows included), a fraction of S
    partition_iters: int = 4  # partitioned mode: Lloyd iterations of each grouping

    @classmethod
    def from_workload(cls, wl) -> "PathConfig":
        return cls(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, S=wl.S, D=wl.D, labels=wl.labels, C=wl.C, scale=wl.scale,
                   mask_mode=wl.mask_mode, keep=wl.mask, block=wl.block, stride=wl.stride,
                   score_scale=wl.score_scale or None, tau=wl.tau, pool_gqa=wl.pool_gqa, compensate=wl.compensate,
                   probes=wl.probes, lam=wl.lam, rank=wl.rank)


@dataclass
class PathResult:
    out: torch.Tensor
    layout: api.ClusterLayout
    mask: api.BlockMask
    scores: Optional[torch.Tensor] = None
    kbar: Optional[torch.Tensor] = None
    vbar: Optional[torch.Tensor] = None
    out_sparse: Optional[torch.Tensor] = None  # rows before the correction (only if requested)
    o_dense_probe: Optional[torch.Tensor] = None
    o_sparse_probe: Optional[torch.Tensor] = None
    A: Optional[torch.Tensor] = None
    c: Optional[torch.Tensor] = None
    extras: dict = field(default_factory=dict)


class SparseAttentionPath:
    """Holds the per-call constants (labels, probe rows, thresholds) on the device."""

    def __init__(self, cfg: PathConfig, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self._pack_buffer = None  # reused across calls
        self._attn_ws = None
        self._side = None  # second stream for the mask-independent stages
        self._scores = None  # score rows kept across calls when a mask cache is used
        self._probe_ws = None  # dense probe partials (bfloat16 inputs)
        self.labels = torch.as_tensor(np.ascontiguousarray(cfg.labels, dtype=np.int32)).to(self.device)
        if cfg.mask_mode not in ("given", "scored", "routed", "partitioned"):
            raise ValueError(f"unknown mask mode {cfg.mask_mode!r}")
        self._err_ws = None  # routed modes: block-error workspace
        self._part_ws = None  # partitioned mode: partition workspace
        if cfg.mask_mode in ("routed", "partitioned"):
            if cfg.D not in (64, 128) or not 0.0 <= cfg.route_density <= 1.0:
                raise ValueError("routed modes need D in {64, 128} and 0 <= route_density <= 1")
        elif cfg.mask_mode == "given":
            keep = np.asarray(cfg.keep, dtype=np.uint8)
            if keep.shape[0] == 1 and cfg.B > 1:
                keep = np.broadcast_to(keep, (cfg.B,) + keep.shape[1:])
            self.given_keep = torch.as_tensor(np.ascontiguousarray(keep)).to(self.device)
        elif cfg.mask_mode == "scored":
            # Score block i covers cluster-major tokens [i*block, (i+1)*block) and its mask row is
            # used as query cluster i's row: every cluster must be exactly one block.
            counts = np.bincount(np.asarray(cfg.labels, dtype=np.int64), minlength=cfg.C)
            nb = -(-cfg.S // cfg.block)
            if (cfg.C != nb or counts.size != cfg.C or np.any(counts[:-1] != cfg.block)
                    or not 1 <= counts[-1] <= cfg.block):
                raise ValueError("scored masks need clusters of exactly `block` tokens (the last one may be "
                                 "shorter): cluster i must be score block i")
            self.tau = torch.as_tensor(np.asarray(cfg.tau, dtype=np.float32).reshape(-1)).to(self.device)
        max_probes = min(_lib.MAX_FIT_PROBES, _lib.MAX_PROBE_ROWS)
        if cfg.probes and not 2 <= cfg.probes <= max_probes:
            raise ValueError(f"probes must lie in [2, {max_probes}] (the probe rows' and the ridge fit's range)")
        if cfg.probes and cfg.mask_mode != "partitioned":
            idx, w = api.select_probe_rows(cfg.labels, cfg.C, cfg.probes)
            self.probe_idx = torch.as_tensor(idx).to(self.device)
            self.probe_w = torch.as_tensor(w).to(self.device)

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep_sparse: bool = False,
                 mark: Optional[Callable[[str], None]] = None,
                 cache: Optional[api.HeadMaskCache] = None) -> PathResult:
        """Run the path.  With probes, the probe rows (dense and block-sparse) and the fit come
        before the attention, whose epilogue writes every corrected row, rounded once;
        keep_sparse also returns the rows without the correction (one more attention call).
        ``mark(stage)`` is called after each stage's launches, with the stage's stream current
        (for stream-ordered timing events; a stage spans from the previous mark on its
        stream).  ``cache`` (scored masks only): head-wise mask reuse across calls -- only the
        heads whose Q/K summaries drifted are scored, and the attention uses the cached mask
        ("Dynamic block masks and head-wise mask reuse", "Recipe"); one cache per layer."""
        cfg = self.cfg
        mark = mark or (lambda name: None)
        if cfg.mask_mode == "partitioned":
            return self._partitioned(q, k, v, keep_sparse, mark)
        main = torch.cuda.current_stream(q.device)
        mark("start")
        layout = api.cluster_layout(self.labels, cfg.C)
        mark("layout")
        side = main
        if cfg.overlap:
            if self._side is None:
                self._side = torch.cuda.Stream(device=q.device)
            side = self._side
            side.wait_stream(main)
        with torch.cuda.stream(side):
            mark("side")
            # One pass over K/V: cluster tiles for the attention kernel and the centroids.
            kv = api.kv_pack(k, v, layout, self._pack_buffer)
            mark("pack")
        if side is not main:
            # Tensors made on the side stream and read on the caller's stream, and the
            # reverse, stay allocated until both streams are past them.
            for t in (kv.buffer, kv.kbar, kv.vbar):
                if t is not None:
                    t.record_stream(main)
            for t in (layout.perm, layout.offsets, layout.counts, q, k, v):
                t.record_stream(side)
        self._pack_buffer = kv.buffer
        kbar, vbar = (kv.kbar, kv.vbar) if cfg.compensate else (None, None)
        scores = None
        if cfg.mask_mode == "scored" and cache is not None:
            Hs = cfg.Hkv if cfg.pool_gqa else cfg.Hq
            if cache.Hm is None:
                cache.Hm = Hs
            if cache.Hm != Hs:
                raise ValueError(f"the cache keeps {cache.Hm} mask heads, the scores have {Hs}")
            refresh = cache.should_refresh(q, k)
            mark("reuse_decide")
            nb = -(-cfg.S // cfg.block)
            if self._scores is None or self._scores.shape != (cfg.B, Hs, nb, nb):
                self._scores = torch.empty(cfg.B, Hs, nb, nb, dtype=torch.float32, device=q.device)
            scores = api.antidiagonal_block_scores(q, k, layout, cfg.block, cfg.stride,
                                                   cfg.score_scale or 1.0 / math.sqrt(cfg.D), cfg.pool_gqa,
                                                   heads=refresh, out=self._scores)
            mark("scores")
            mask = cache.update(api.top_p_block_mask(scores, self.tau), refresh)
            mark("top_p")
        elif cfg.mask_mode == "scored":
            scores = api.antidiagonal_block_scores(q, k, layout, cfg.block, cfg.stride,
                                                   cfg.score_scale or 1.0 / math.sqrt(cfg.D), cfg.pool_gqa)
            mark("scores")
            mask = api.top_p_block_mask(scores, self.tau)
            mark("top_p")
        elif cfg.mask_mode == "routed":
            # Error-aware routes need the packed tiles and centroids: wait for the pack.
            if side is not main:
                main.wait_stream(side)
            qbar = api.query_centroids(q, layout)
            mark("route_probes")
            if self._err_ws is None:
                n = _lib.size_query("bsa_block_error_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D, cfg.C,
                                    cfg.C)
                self._err_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
            err = api.block_error(qbar, kv, cfg.scale, workspace=self._err_ws)
            mark("block_error")
            mask = api.error_route(err, layout, int(round(cfg.route_density * cfg.S)))
            mark("route")
        else:
            mask = api.mask_from_keep(self.given_keep)
            mark("mask_lists")
        if side is not main:
            main.wait_stream(side)
        mark("join")
        res = PathResult(out=None, layout=layout, mask=mask, scores=scores, kbar=kbar, vbar=vbar)
        if self._attn_ws is None:
            self._attn_ws = api.attention_workspace(q, kv, layout, mask)
        if not cfg.probes:
            res.out = api.block_sparse_attention(q, kv, layout, mask, cfg.compensate, cfg.scale,
                                                 workspace=self._attn_ws)
            mark("attention")
            return res
        # Fit before attending: the probes' dense and block-sparse rows (one pass over the packed
        # tiles, float32), the ridge fit, then the attention applies o + o A + c to every row
        # in its epilogue and rounds each row once.
        if q.dtype == torch.bfloat16:
            if self._probe_ws is None:
                n = _lib.size_query("bsa_probe_attention_packed_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S,
                                    cfg.D, cfg.probes, cfg.C)
                self._probe_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
            od, os_ = api.probe_attention_packed(q, kv, self.probe_idx, cfg.scale, workspace=self._probe_ws,
                                                 q_labels=self.labels, mask=mask, compensate=cfg.compensate)
        else:
            od, os_ = api.probe_attention(q, k, v, self.probe_idx, cfg.scale, q_labels=self.labels,
                                          k_labels=self.labels, k_layout=layout, mask=mask, kbar=kbar, vbar=vbar)
        mark("probe_rows")
        A, c = api.probe_fit(os_, od, self.probe_w, cfg.lam, cfg.rank)
        mark("fit")
        res.out = api.block_sparse_attention(q, kv, layout, mask, cfg.compensate, cfg.scale, workspace=self._attn_ws,
                                             A=A, c=c)
        mark("attention")
        res.o_dense_probe, res.o_sparse_probe, res.A, res.c = od, os_, A, c
        if keep_sparse:  # the uncorrected rows too (an extra attention call, for inspection)
            res.out_sparse = api.block_sparse_attention(q, kv, layout, mask, cfg.compensate, cfg.scale,
                                                        workspace=self._attn_ws)
        return res

    def _partitioned(self, q, k, v, keep_sparse, mark) -> PathResult:
        """SparsePR's call ("Partition the Support, Reconstruct the Residual": partitioning,
        routing, permutation, the sparse kernel, probes, the fit and write-back all inside the
        call): response-coupled key and query groups per (batch, K/V head), their layouts, the
        packed K/V, error-aware routes (the probe rows' cost reserved from the density target
        first), then -- with probes -- the probes of every layout, their dense and sparse rows
        and the fit, and the compensated attention with the correction in its epilogue."""
        cfg = self.cfg
        mark("start")
        if q.dtype != torch.bfloat16:
            raise ValueError("the partitioned path routes with block errors, which take bfloat16 inputs")
        if self._part_ws is None:
            n = _lib.size_query("bsa_response_partition_workspace_size", cfg.B, cfg.Hkv, cfg.S, cfg.D, cfg.C, cfg.C)
            self._part_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
        k_labels, q_labels = api.response_partition(q, k, cfg.C, cfg.C, cfg.scale, iters=cfg.partition_iters,
                                                    workspace=self._part_ws)
        mark("partition")
        klay = api.cluster_layout(k_labels, cfg.C)
        qlay = api.cluster_layout(q_labels, cfg.C)
        mark("layout")
        kv = api.kv_pack(k, v, klay, self._pack_buffer)
        self._pack_buffer = kv.buffer
        mark("pack")
        qbar = api.query_centroids(q, qlay)
        mark("route_probes")
        if self._err_ws is None:
            n = _lib.size_query("bsa_block_error_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D, cfg.C, cfg.C)
            self._err_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
        err = api.block_error(qbar, kv, cfg.scale, workspace=self._err_ws)
        mark("block_error")
        # Executed-pair density = routing density + M / S: the probe rows' share comes first.
        budget = max(0, int(round(cfg.route_density * cfg.S)) - cfg.probes)
        mask = api.error_route(err, klay, budget)
        mark("route")
        res = PathResult(out=None, layout=klay, mask=mask, kbar=kv.kbar if cfg.compensate else None,
                         vbar=kv.vbar if cfg.compensate else None)
        res.extras.update(q_layout=qlay, k_labels=k_labels, q_labels=q_labels, budget=budget)
        if self._attn_ws is None:
            self._attn_ws = api.attention_workspace(q, kv, qlay, mask)
        A = c = None
        if cfg.probes:
            pidx, pw = api.select_probe_rows_layouts(qlay, cfg.probes)
            mark("probe_select")
            if self._probe_ws is None:
                n = _lib.size_query("bsa_probe_attention_packed_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S,
                                    cfg.D, cfg.probes, cfg.C)
                self._probe_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
            od, os_ = api.probe_attention_packed(q, kv, pidx, cfg.scale, workspace=self._probe_ws,
                                                 q_labels=q_labels.reshape(-1, cfg.S), mask=mask,
                                                 compensate=cfg.compensate)
            mark("probe_rows")
            A, c = api.probe_fit(os_, od, pw, cfg.lam, cfg.rank)
            mark("fit")
            res.o_dense_probe, res.o_sparse_probe, res.A, res.c = od, os_, A, c
            res.extras.update(probe_idx=pidx, probe_w=pw)
        res.out = api.block_sparse_attention(q, kv, qlay, mask, cfg.compensate, cfg.scale, workspace=self._attn_ws,
                                             A=A, c=c)
        mark("attention")
        if keep_sparse and A is not None:
            res.out_sparse = api.block_sparse_attention(q, kv, qlay, mask, cfg.compensate, cfg.scale,
                                                        workspace=self._attn_ws)
        return res
