"""The whole path as one call: layout -> centroids -> scores -> top-p -> sparse attention
-> probe rows -> fit -> correction.

Order of stages: "Dynamic block masks and head-wise mask reuse", section "Recipe" (scores,
top-p mask, labels, compensated attention) and "Sparse-block compensation", section
"Recipe: STA with both repairs" (compensated attention, probe selection, dense probe rows,
residual correction).  Every stage is one or two kernel launches on the current stream;
nothing is computed on the host except the probe selection, which depends only on the
labels and is done once.

Streams: the K/V packing and the dense probe rows depend only on the inputs and the layout,
so they run on a second stream (default priority) while the scores and the top-p masks run
on the caller's stream; the attention waits for both.
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
    labels: np.ndarray  # int32 [S] (host)
    C: int
    scale: float
    mask_mode: str  # "given", "scored" or "routed" (error-aware routes under route_density)
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
    overlap: bool = True  # pack and probe rows on a second stream, beside scores and top-p
    route_density: float = 0.2  # routed mode: keys each row computes exactly, as a fraction of S

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
    out_sparse: Optional[torch.Tensor] = None  # float32 rows before the correction (only if requested)
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
        self._o32 = None  # float32 attention rows before the correction
        self._side = None  # second stream for the mask-independent stages
        self._scores = None  # score rows kept across calls when a mask cache is used
        self._probe_ws = None  # dense probe partials (bfloat16 inputs)
        self.labels = torch.as_tensor(np.ascontiguousarray(cfg.labels, dtype=np.int32)).to(self.device)
        if cfg.mask_mode not in ("given", "scored", "routed"):
            raise ValueError(f"unknown mask mode {cfg.mask_mode!r}")
        self._err_ws = None  # routed mode: block-error workspace
        if cfg.mask_mode == "routed":
            if cfg.D not in (64, 128) or not 0.0 <= cfg.route_density <= 1.0:
                raise ValueError("routed mode needs D in {64, 128} and 0 <= route_density <= 1")
        elif cfg.mask_mode == "given":
            keep = np.asarray(cfg.keep, dtype=np.uint8)
            if keep.shape[0] == 1 and cfg.B > 1:
                keep = np.broadcast_to(keep, (cfg.B,) + keep.shape[1:])
            self.given_keep = torch.as_tensor(np.ascontiguousarray(keep)).to(self.device)
        elif cfg.mask_mode == "scored":
            self.tau = torch.as_tensor(np.asarray(cfg.tau, dtype=np.float32).reshape(-1)).to(self.device)
        if cfg.probes:
            idx, w = api.select_probe_rows(cfg.labels, cfg.C, cfg.probes)
            self.probe_idx = torch.as_tensor(idx).to(self.device)
            self.probe_w = torch.as_tensor(w).to(self.device)

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep_sparse: bool = False,
                 mark: Optional[Callable[[str], None]] = None,
                 cache: Optional[api.HeadMaskCache] = None) -> PathResult:
        """Run the path.  With probes the attention keeps its rows in float32, the fit reads
        the probe rows from them, and the correction pass writes every corrected row, rounded
        once; keep_sparse also returns the float32 rows before the correction.
        ``mark(stage)`` is called after each stage's launches, with the stage's stream current
        (for stream-ordered timing events; a stage spans from the previous mark on its
        stream).  ``cache`` (scored masks only): head-wise mask reuse across calls -- only the
        heads whose Q/K summaries drifted are scored, and the attention uses the cached mask
        ("Dynamic block masks and head-wise mask reuse", "Recipe"); one cache per layer."""
        cfg = self.cfg
        mark = mark or (lambda name: None)
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
            od = None
            if cfg.probes:  # exact dense probe rows: independent of the mask
                if q.dtype == torch.bfloat16:  # from the packed tiles just written
                    if self._probe_ws is None:
                        n = _lib.size_query("bsa_probe_attention_packed_workspace_size", cfg.B, cfg.Hq, cfg.Hkv,
                                            cfg.S, cfg.D, cfg.probes, cfg.C)
                        self._probe_ws = torch.empty(n, dtype=torch.uint8, device=q.device)
                    od = api.probe_attention_packed(q, kv, self.probe_idx, cfg.scale, workspace=self._probe_ws)
                else:
                    od, _ = api.probe_attention(q, k, v, self.probe_idx, cfg.scale)
                mark("probe_rows")
        if side is not main:
            # Tensors made on the side stream and read on the caller's stream, and the
            # reverse, stay allocated until both streams are past them.
            for t in (kv.buffer, kv.kbar, kv.vbar, od):
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
        if self._o32 is None or self._o32.shape != q.shape:
            self._o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o32 = api.block_sparse_attention(q, kv, layout, mask, cfg.compensate, cfg.scale, out=self._o32, out_f32=True,
                                         workspace=self._attn_ws)
        mark("attention")
        os_ = api.gather_rows(o32, self.probe_idx)
        A, c = api.probe_fit(os_, od, self.probe_w, cfg.lam, cfg.rank)
        mark("fit")
        res.out = api.correct(o32, A, c, q.dtype)
        mark("correct")
        res.o_dense_probe, res.o_sparse_probe, res.A, res.c = od, os_, A, c
        if keep_sparse:
            res.out_sparse = o32.clone()
        return res
