"""Torch-tensor front end of the C ABI (argument marshalling only).

Every function checks shapes, dtypes and devices, allocates its outputs with torch on the
current device, and calls the matching ``bsa_*`` entry point on torch's current stream.
All arithmetic happens in the HIP kernels.  Names follow the pages' API (Sparse-block
compensation, API table; Dynamic block masks and head-wise mask reuse, API table).
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import BSA_BF16, BSA_F32


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


@dataclass
class ClusterLayout:
    """Cluster-major order of tokens: cluster c owns perm[offsets[c]:offsets[c+1]]."""

    perm: torch.Tensor  # int32 [S], or [P, S] for P layouts
    offsets: torch.Tensor  # int32 [C+1] or [P, C+1]
    counts: torch.Tensor  # int32 [C] or [P, C]
    C: int

    @property
    def n_layouts(self) -> int:
        """1 for one layout shared by every head, else the number of layouts (B * Hkv: one per
        (batch, K/V head), layout b * Hkv + kvh)."""
        return 1 if self.perm.dim() == 1 else int(self.perm.shape[0])


def cluster_layout(labels: torch.Tensor, C: int) -> ClusterLayout:
    """Stable counting sort of int32 labels in [0, C) (bsa_cluster_layout): labels [S] give one
    layout; labels [..., S] (e.g. [B, Hkv, S] from response_partition) give one per leading
    index, flattened to [P, S]."""
    _check_cuda(labels)
    if labels.dtype != torch.int32 or labels.dim() < 1:
        raise ValueError("labels must be int32 [S] or [..., S]")
    S = labels.shape[-1]
    P = labels.numel() // S
    dev = labels.device
    lead = () if labels.dim() == 1 else (P,)
    perm = torch.empty(*lead, S, dtype=torch.int32, device=dev)
    offsets = torch.empty(*lead, C + 1, dtype=torch.int32, device=dev)
    counts = torch.empty(*lead, C, dtype=torch.int32, device=dev)
    nbytes = _lib.size_query("bsa_cluster_layout_workspace_size", P, S, C)
    ws = _workspace(nbytes, dev)
    _lib.call("bsa_cluster_layout", P, _ptr(labels.contiguous()), S, C, _ptr(perm), _ptr(offsets), _ptr(counts),
              _ptr(ws), ws.numel(), _stream())
    return ClusterLayout(perm, offsets, counts, C)


def select_probe_rows_layouts(layout: ClusterLayout, M: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Probe rows and weights of every layout on the device (bsa_select_probe_rows_layouts):
    int32 [P, M] and float32 [P, M]."""
    perm = layout.perm if layout.perm.dim() == 2 else layout.perm[None]
    P, S = perm.shape
    idx = torch.empty(P, M, dtype=torch.int32, device=perm.device)
    w = torch.empty(P, M, dtype=torch.float32, device=perm.device)
    _lib.call("bsa_select_probe_rows_layouts", P, S, layout.C, int(M), _ptr(perm), _ptr(layout.offsets), _ptr(idx),
              _ptr(w), _stream())
    return idx, w


def centroids(k: torch.Tensor, v: torch.Tensor, layout: ClusterLayout) -> Tuple[torch.Tensor, torch.Tensor]:
    """Key/value cluster means, float32 [B, Hkv, C, D] (bsa_centroids)."""
    _check_cuda(k, v)
    B, Hkv, S, D = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must match")
    kbar = torch.empty(B, Hkv, layout.C, D, dtype=torch.float32, device=k.device)
    vbar = torch.empty_like(kbar)
    _lib.call("bsa_centroids", B, Hkv, S, D, _dtype_code(k), _ptr(k), _ptr(v), _ptr(layout.perm),
              _ptr(layout.offsets), layout.C, _ptr(kbar), _ptr(vbar), _stream())
    return kbar, vbar


@dataclass
class PackedKV:
    """Keys and values in cluster-major 64-key tiles plus the centroid tiles (bsa_kv_pack).
    ``buffer`` is opaque; it belongs to ``layout`` and the K/V shape it was packed from."""

    buffer: torch.Tensor  # uint8
    kbar: torch.Tensor  # float32 [B, Hkv, C, D]
    vbar: torch.Tensor  # float32 [B, Hkv, C, D]
    layout: ClusterLayout
    B: int
    Hkv: int
    S: int
    D: int
    dtype: torch.dtype


def kv_pack(k: torch.Tensor, v: torch.Tensor, layout: ClusterLayout,
            buffer: Optional[torch.Tensor] = None) -> PackedKV:
    """Pack K/V into cluster tiles and compute the cluster means (bsa_kv_pack)."""
    _check_cuda(k, v)
    B, Hkv, S, D = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must match")
    code = _dtype_code(k)
    nl = layout.n_layouts
    nbytes = _lib.size_query("bsa_kv_pack_workspace_size", B, Hkv, S, D, code, layout.C, nl)
    if buffer is None or buffer.numel() < nbytes:
        buffer = _workspace(nbytes, k.device)
    kbar = torch.empty(B, Hkv, layout.C, D, dtype=torch.float32, device=k.device)
    vbar = torch.empty_like(kbar)
    _lib.call("bsa_kv_pack", B, Hkv, S, D, code, _ptr(k), _ptr(v), _ptr(layout.perm), _ptr(layout.offsets),
              layout.C, nl, _ptr(kbar), _ptr(vbar), _ptr(buffer), buffer.numel(), _stream())
    return PackedKV(buffer, kbar, vbar, layout, B, Hkv, S, D, k.dtype)


def kv_pack_centroids(k: torch.Tensor, v: torch.Tensor, layout: ClusterLayout, kbar: torch.Tensor,
                      vbar: torch.Tensor, counts: torch.Tensor, buffer: Optional[torch.Tensor] = None) -> PackedKV:
    """Pack K/V into cluster tiles with the caller's centroids kbar, vbar (float32 [B, Hkv, C, D])
    and counts (int32 [C], or [P, C] with P layouts: the n_c of each centroid column)
    (bsa_kv_pack_centroids)."""
    _check_cuda(k, v, kbar, vbar, counts)
    B, Hkv, S, D = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must match")
    if kbar.shape != (B, Hkv, layout.C, D) or vbar.shape != kbar.shape or kbar.dtype != torch.float32 \
            or vbar.dtype != torch.float32:
        raise ValueError("kbar and vbar must be float32 [B, Hkv, C, D]")
    nl = layout.n_layouts
    if counts.shape != layout.counts.shape or counts.dtype != torch.int32:
        raise ValueError("counts must be int32 [C] (or [P, C] for P layouts)")
    code = _dtype_code(k)
    nbytes = _lib.size_query("bsa_kv_pack_workspace_size", B, Hkv, S, D, code, layout.C, nl)
    if buffer is None or buffer.numel() < nbytes:
        buffer = _workspace(nbytes, k.device)
    _lib.call("bsa_kv_pack_centroids", B, Hkv, S, D, code, _ptr(k), _ptr(v), _ptr(layout.perm),
              _ptr(layout.offsets), layout.C, nl, _ptr(kbar), _ptr(vbar), _ptr(counts), _ptr(buffer),
              buffer.numel(), _stream())
    return PackedKV(buffer, kbar, vbar, layout, B, Hkv, S, D, k.dtype)


def antidiagonal_block_scores(q: torch.Tensor, k: torch.Tensor, layout: Optional[ClusterLayout] = None,
                              block_size: int = 128, stride: int = 16, score_scale: Optional[float] = None,
                              pool_gqa: bool = False, workspace: Optional[torch.Tensor] = None,
                              heads: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Normalized antidiagonal block scores [B, Hs, nb, nb] (bsa_antidiag_scores).  With
    ``heads`` (uint8 [B, Hs]) only the flagged heads are scored (bsa_antidiag_scores_heads);
    the other rows of ``out`` are left as they were."""
    _check_cuda(q, k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k shapes/dtypes do not match")
    if score_scale is None:
        score_scale = 1.0 / math.sqrt(D)
    nb = -(-S // block_size)
    Hs = Hkv if pool_gqa else Hq
    if out is not None:
        _check_cuda(out)
        if out.shape != (B, Hs, nb, nb) or out.dtype != torch.float32:
            raise ValueError("out must be float32 [B, Hs, nb, nb]")
        scores = out
    else:
        scores = torch.empty(B, Hs, nb, nb, dtype=torch.float32, device=q.device)
    nbytes = _lib.size_query("bsa_antidiag_scores_workspace_size", B, Hq, Hkv, S, D, block_size, stride)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    perm = _ptr(layout.perm) if layout is not None else None
    if heads is None:
        _lib.call("bsa_antidiag_scores", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(k), perm, block_size, stride,
                  float(score_scale), int(pool_gqa), _ptr(scores), _ptr(workspace), workspace.numel(), _stream())
    else:
        _check_cuda(heads)
        if heads.dtype != torch.uint8 or heads.shape != (B, Hs):
            raise ValueError("heads must be uint8 [B, Hs]")
        _lib.call("bsa_antidiag_scores_heads", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(k), perm, block_size,
                  stride, float(score_scale), int(pool_gqa), _ptr(heads), _ptr(scores), _ptr(workspace),
                  workspace.numel(), _stream())
    return scores


@dataclass
class BlockMask:
    """Keep bits [B, Hm, Cq, Ck] and the ascending kept-block list of every row."""

    keep: torch.Tensor  # uint8
    kv_count: torch.Tensor  # int32 [B, Hm, Cq]
    kv_idx: torch.Tensor  # int16 [B, Hm, Cq, Ck]

    @property
    def Hm(self) -> int:
        return int(self.keep.shape[1])


def top_p_block_mask(scores: torch.Tensor, tau) -> BlockMask:
    """Per-row top-p keep bits from scores [B, Hs, Cq, Ck]; tau scalar or [Hs] (bsa_top_p_mask)."""
    _check_cuda(scores)
    B, Hs, Cq, Ck = scores.shape
    if isinstance(tau, torch.Tensor):
        tau_t = tau.to(device=scores.device, dtype=torch.float32).reshape(-1).contiguous()
    else:
        tau_t = torch.as_tensor(np.asarray(tau, dtype=np.float32).reshape(-1)).to(scores.device)
    if tau_t.numel() not in (1, Hs):
        raise ValueError("tau must be a scalar or one value per head")
    keep = torch.empty(B, Hs, Cq, Ck, dtype=torch.uint8, device=scores.device)
    cnt = torch.empty(B, Hs, Cq, dtype=torch.int32, device=scores.device)
    idx = torch.empty(B, Hs, Cq, Ck, dtype=torch.int16, device=scores.device)
    _lib.call("bsa_top_p_mask", _ptr(scores), B * Hs, Cq, Ck, _ptr(tau_t), tau_t.numel(), Hs, _ptr(keep), _ptr(cnt),
              _ptr(idx), _stream())
    return BlockMask(keep, cnt, idx)


def mask_from_keep(keep: torch.Tensor) -> BlockMask:
    """Kept-block lists of a caller-given uint8 mask [B, Hm, Cq, Ck] (bsa_mask_lists)."""
    keep = keep.to(torch.uint8).contiguous()
    _check_cuda(keep)
    B, Hm, Cq, Ck = keep.shape
    cnt = torch.empty(B, Hm, Cq, dtype=torch.int32, device=keep.device)
    idx = torch.empty(B, Hm, Cq, Ck, dtype=torch.int16, device=keep.device)
    _lib.call("bsa_mask_lists", _ptr(keep), B * Hm * Cq, Ck, _ptr(cnt), _ptr(idx), _stream())
    return BlockMask(keep, cnt, idx)


def _layout_count(q_layout: ClusterLayout, kv: PackedKV) -> int:
    """The layout count of a call: the query and key layouts must have the same (1, or one per
    (batch, K/V head))."""
    nl = kv.layout.n_layouts
    if q_layout.n_layouts != nl or nl not in (1, kv.B * kv.Hkv):
        raise ValueError("query and key layouts must both be shared, or both one per (batch, K/V head)")
    return nl


def block_sparse_attention(q: torch.Tensor, kv: PackedKV, q_layout: ClusterLayout, mask: BlockMask,
                           compensate: bool = True, scale: Optional[float] = None, return_lse: bool = False,
                           out: Optional[torch.Tensor] = None, out_f32: bool = False,
                           workspace: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                           c: Optional[torch.Tensor] = None):
    """Block-sparse attention over packed K/V; compensated by the skipped clusters'
    centroids, or hard drop with compensate=False (bsa_sparse_attention).  With out_f32 the
    rows are returned in float32 (for a later correction, see correct).  With A, c (from
    probe_fit) every row o is written as o + o A + c, rounded once (the repair epilogue)."""
    _check_cuda(q, out, A, c)
    if (A is None) != (c is None):
        raise ValueError("A and c go together")
    if A is not None:
        if out_f32:
            raise ValueError("the repair epilogue writes the input type")
        if A.shape != (q.shape[0], q.shape[1], q.shape[3], q.shape[3]) or c.shape != (q.shape[0], q.shape[1], q.shape[3]) \
                or A.dtype != torch.float32 or c.dtype != torch.float32:
            raise ValueError("A must be float32 [B, Hq, D, D] and c float32 [B, Hq, D]")
    B, Hq, S, D = q.shape
    if (kv.B, kv.S, kv.D, kv.dtype) != (B, S, D, q.dtype) or Hq % kv.Hkv != 0:
        raise ValueError("q does not match the packed K/V")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Ck = kv.layout.C
    if mask.keep.shape[0] != B or mask.keep.shape[2] != q_layout.C or mask.keep.shape[3] != Ck:
        raise ValueError("mask shape does not match batch / cluster counts")
    odt = torch.float32 if out_f32 else q.dtype
    o = torch.empty(B, Hq, S, D, dtype=odt, device=q.device) if out is None else out
    if o.dtype != odt or o.shape != q.shape:
        raise ValueError("out has the wrong shape or dtype")
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device) if return_lse else None
    nl = _layout_count(q_layout, kv)
    nbytes = _lib.size_query("bsa_sparse_attention_workspace_size", B, Hq, mask.Hm, q_layout.C, S, Ck)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    _lib.call("bsa_sparse_attention", B, Hq, kv.Hkv, S, D, _dtype_code(q), _ptr(q), float(scale),
              _ptr(q_layout.perm), _ptr(q_layout.offsets), q_layout.C, _ptr(kv.layout.offsets), Ck, nl,
              _ptr(mask.keep), _ptr(mask.kv_count), _ptr(mask.kv_idx), mask.Hm, _ptr(kv.buffer), kv.buffer.numel(),
              int(bool(compensate)), _ptr(A), _ptr(c), _dtype_code(o), _ptr(o), _ptr(lse), _ptr(workspace),
              workspace.numel(), _stream())
    return (o, lse) if return_lse else o


def block_sparse_attention_noalloc(q: torch.Tensor, kv: PackedKV, q_layout: ClusterLayout, mask: BlockMask,
                                   out: torch.Tensor, compensate: bool = True, scale: Optional[float] = None,
                                   A: Optional[torch.Tensor] = None, c: Optional[torch.Tensor] = None,
                                   lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """block_sparse_attention without a workspace (bsa_sparse_attention_noalloc): the library's
    static device scratch serves the call and nothing is allocated, so `out` (and `lse` if
    wanted) must be given.  Calls that overlap on one GPU race (they share the scratch)."""
    _check_cuda(q, out, A, c, lse)
    B, Hq, S, D = q.shape
    if (kv.B, kv.S, kv.D, kv.dtype) != (B, S, D, q.dtype) or Hq % kv.Hkv != 0:
        raise ValueError("q does not match the packed K/V")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Ck = kv.layout.C
    if mask.keep.shape[0] != B or mask.keep.shape[2] != q_layout.C or mask.keep.shape[3] != Ck:
        raise ValueError("mask shape does not match batch / cluster counts")
    if out.shape != q.shape or out.dtype not in (q.dtype, torch.float32):
        raise ValueError("out has the wrong shape or dtype")
    _lib.call("bsa_sparse_attention_noalloc", B, Hq, kv.Hkv, S, D, _dtype_code(q), _ptr(q), float(scale),
              _ptr(q_layout.perm), _ptr(q_layout.offsets), q_layout.C, _ptr(kv.layout.offsets), Ck,
              _layout_count(q_layout, kv), _ptr(mask.keep), _ptr(mask.kv_count), _ptr(mask.kv_idx), mask.Hm, _ptr(kv.buffer), kv.buffer.numel(),
              int(bool(compensate)), _ptr(A), _ptr(c), _dtype_code(out), _ptr(out), _ptr(lse), _stream())
    return out


def correct(o32: torch.Tensor, A: torch.Tensor, c: torch.Tensor, dtype: torch.dtype = torch.bfloat16,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Every row o of the float32 output becomes o + o A + c, rounded once to dtype (bsa_correct)."""
    _check_cuda(o32, A, c, out)
    if o32.dtype != torch.float32:
        raise ValueError("o32 must be float32")
    B, Hq, S, D = o32.shape
    o = torch.empty(B, Hq, S, D, dtype=dtype, device=o32.device) if out is None else out
    code = BSA_BF16 if o.dtype == torch.bfloat16 else BSA_F32
    _lib.call("bsa_correct", B, Hq, S, D, code, _ptr(o32), _ptr(A), _ptr(c), _ptr(o), _stream())
    return o


def gather_rows(x: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """Rows idx of float32 x [B, H, S, D] -> [B, H, M, D] (bsa_gather_rows)."""
    _check_cuda(x, idx)
    B, H, S, D = x.shape
    M = idx.numel()
    out = torch.empty(B, H, M, D, dtype=torch.float32, device=x.device)
    _lib.call("bsa_gather_rows", B * H, S, D, _ptr(x), _ptr(idx), M, _ptr(out), _stream())
    return out


def attention_workspace(q: torch.Tensor, kv: PackedKV, q_layout: ClusterLayout, mask: BlockMask) -> torch.Tensor:
    """Workspace for block_sparse_attention (the mask rows' tile lists), for reuse across calls."""
    B, Hq, S, _ = q.shape
    nbytes = _lib.size_query("bsa_sparse_attention_workspace_size", B, Hq, mask.Hm, q_layout.C, S, kv.layout.C)
    return _workspace(nbytes, q.device)


def centroid_compensated_attention(q, k, v, q_layout: ClusterLayout, k_layout: ClusterLayout, mask: BlockMask,
                                   compensate: bool = True, scale: Optional[float] = None, return_lse: bool = False,
                                   out: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                                   c: Optional[torch.Tensor] = None, kbar: Optional[torch.Tensor] = None,
                                   vbar: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None):
    """The pages' compensated attention for callers holding plain K/V ("Sparse-block
    compensation", API table): packs K/V (with the caller's centroids kbar, vbar and counts
    when given, else the clusters' means and sizes) and runs block_sparse_attention; with A, c
    every output row o becomes o + o A + c before it is rounded (the repair epilogue)."""
    if kbar is not None or vbar is not None or counts is not None:
        kv = kv_pack_centroids(k, v, k_layout, kbar, vbar, counts)
    else:
        kv = kv_pack(k, v, k_layout)
    return block_sparse_attention(q, kv, q_layout, mask, compensate, scale, return_lse, out, A=A, c=c)


def probe_attention(q, k, v, probe_idx: torch.Tensor, scale: Optional[float] = None,
                    q_labels: Optional[torch.Tensor] = None, k_labels: Optional[torch.Tensor] = None,
                    k_layout: Optional[ClusterLayout] = None, mask: Optional[BlockMask] = None,
                    kbar: Optional[torch.Tensor] = None, vbar: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Probe rows in float32 [B, Hq, M, D]: exact dense rows, and (when a mask is given) the
    same rows under the block-sparse rule (bsa_probe_attention).  Returns (dense, sparse)."""
    _check_cuda(q, k, v, probe_idx, q_labels, k_labels, kbar, vbar)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    M = probe_idx.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    od = torch.empty(B, Hq, M, D, dtype=torch.float32, device=q.device)
    os_ = torch.empty_like(od) if mask is not None else None
    nbytes = _lib.size_query("bsa_probe_attention_workspace_size", B, Hq, S, D, M)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    if mask is not None:
        Hm, Cq, Ck = mask.Hm, int(mask.keep.shape[2]), int(mask.keep.shape[3])
        args = (_ptr(q_labels), _ptr(k_labels), _ptr(mask.keep), Hm, Cq, Ck, _ptr(k_layout.offsets), _ptr(kbar),
                _ptr(vbar))
    else:
        args = (None, None, None, 1, 1, 1, None, None, None)
    _lib.call("bsa_probe_attention", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), float(scale),
              _ptr(probe_idx), M, *args, _ptr(od), _ptr(os_), _ptr(workspace), workspace.numel(), _stream())
    return od, os_


def probe_attention_packed(q: torch.Tensor, kv: PackedKV, probe_idx: torch.Tensor, scale: Optional[float] = None,
                           workspace: Optional[torch.Tensor] = None, q_labels: Optional[torch.Tensor] = None,
                           mask: Optional[BlockMask] = None, compensate: bool = True):
    """Probe rows, float32 [B, Hq, M, D], from the packed K/V tiles of kv_pack (bfloat16 inputs;
    bsa_probe_attention_packed): the exact dense rows, and with q_labels and a mask also the
    same rows under the block-sparse rule (compensated or hard drop), from the same pass.
    Returns the dense rows, or (dense, sparse) when a mask is given."""
    _check_cuda(q, probe_idx, q_labels)
    B, Hq, S, D = q.shape
    if (kv.B, kv.S, kv.D, kv.dtype) != (B, S, D, q.dtype) or Hq % kv.Hkv != 0:
        raise ValueError("packed K/V do not match q")
    nl = kv.layout.n_layouts
    M = probe_idx.shape[-1]
    if probe_idx.numel() != (nl if nl > 1 else 1) * M:
        raise ValueError("probe_idx must be [M], or [P, M] with the P layouts of kv")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    od = torch.empty(B, Hq, M, D, dtype=torch.float32, device=q.device)
    os_ = torch.empty_like(od) if mask is not None else None
    C = kv.layout.C
    nbytes = _lib.size_query("bsa_probe_attention_packed_workspace_size", B, Hq, kv.Hkv, S, D, M, C)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    if mask is not None:
        if q_labels is None or mask.keep.shape[0] != B or mask.keep.shape[3] != C:
            raise ValueError("sparse probe rows need the query labels and a [B, Hm, Cq, Ck] mask")
        sargs = (_ptr(q_labels), _ptr(mask.keep), mask.Hm, int(mask.keep.shape[2]), int(bool(compensate)))
    else:
        sargs = (None, None, 1, 1, 0)
    _lib.call("bsa_probe_attention_packed", B, Hq, kv.Hkv, S, D, _dtype_code(q), _ptr(q), float(scale),
              _ptr(probe_idx), M, _ptr(kv.buffer), kv.buffer.numel(), _ptr(kv.layout.offsets), C, nl, *sargs,
              _ptr(od), _ptr(os_), _ptr(workspace), workspace.numel(), _stream())
    return od if mask is None else (od, os_)


def query_centroids(q: torch.Tensor, layout: ClusterLayout, Hkv: Optional[int] = None) -> torch.Tensor:
    """Mean query row of every query cluster [B, Hq, Cq, D], rounded to q's dtype: the
    probes of the error-aware router (bsa_query_centroids).  With one layout per (batch,
    K/V head) the query heads of K/V head kvh use layout b * Hkv + kvh."""
    _check_cuda(q)
    B, Hq, S, D = q.shape
    nl = layout.n_layouts
    if Hkv is None:
        Hkv = Hq if nl == 1 else nl // B
    out = torch.empty(B, Hq, layout.C, D, dtype=q.dtype, device=q.device)
    _lib.call("bsa_query_centroids", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(layout.perm),
              _ptr(layout.offsets), layout.C, nl, _ptr(out), _stream())
    return out


def block_error(qbar: torch.Tensor, kv: PackedKV, scale: Optional[float] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Compensation error of every block, float32 [B, Hq, Cq, Ck], for the probes qbar
    [B, Hq, Cq, D] against the packed keys and values (bfloat16; bsa_block_error)."""
    _check_cuda(qbar)
    B, Hq, Cq, D = qbar.shape
    if (kv.B, kv.D, kv.dtype) != (B, D, qbar.dtype) or Hq % kv.Hkv != 0:
        raise ValueError("packed K/V do not match qbar")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Ck = kv.layout.C
    err = torch.empty(B, Hq, Cq, Ck, dtype=torch.float32, device=qbar.device)
    nbytes = _lib.size_query("bsa_block_error_workspace_size", B, Hq, kv.Hkv, kv.S, D, Cq, Ck)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, qbar.device)
    _lib.call("bsa_block_error", B, Hq, kv.Hkv, kv.S, D, _dtype_code(qbar), _ptr(qbar), Cq, float(scale),
              _ptr(kv.buffer), kv.buffer.numel(), _ptr(kv.layout.offsets), Ck, kv.layout.n_layouts, _ptr(kv.kbar),
              _ptr(kv.vbar), _ptr(err), _ptr(workspace), workspace.numel(), _stream())
    return err


def error_route(err: torch.Tensor, k_layout: ClusterLayout, budget: int) -> BlockMask:
    """Error-aware routes from block errors [B, H, Cq, Ck]: per row the clusters by err / n_c
    until `budget` key tokens are kept (bsa_error_route)."""
    _check_cuda(err)
    B, H, Cq, Ck = err.shape
    keep = torch.empty(B, H, Cq, Ck, dtype=torch.uint8, device=err.device)
    cnt = torch.empty(B, H, Cq, dtype=torch.int32, device=err.device)
    idx = torch.empty(B, H, Cq, Ck, dtype=torch.int16, device=err.device)
    nl = k_layout.n_layouts
    rows_per_layout = 0 if nl == 1 else (B * H * Cq) // nl  # rows of [B, H, Cq] by (batch, K/V head)
    _lib.call("bsa_error_route", _ptr(err), B * H * Cq, Ck, _ptr(k_layout.offsets), rows_per_layout, int(budget),
              _ptr(keep), _ptr(cnt), _ptr(idx), _stream())
    return BlockMask(keep, cnt, idx)


def probe_fit(o_sparse_probe: torch.Tensor, o_dense_probe: torch.Tensor, weights: torch.Tensor,
              lam: float = 0.1, rank: int = 16) -> Tuple[torch.Tensor, torch.Tensor]:
    """Folded correction map A [B, Hq, D, D], c [B, Hq, D] from float32 probe rows (bsa_probe_fit).
    weights: [M] for every head, or [B * Hkv, M] for probes chosen per (batch, K/V head)."""
    _check_cuda(o_sparse_probe, o_dense_probe, weights)
    B, Hq, M, D = o_sparse_probe.shape
    nl = 1 if weights.dim() == 1 else int(weights.shape[0])
    Hkv = Hq if nl == 1 else nl // B
    A = torch.empty(B, Hq, D, D, dtype=torch.float32, device=o_sparse_probe.device)
    c = torch.empty(B, Hq, D, dtype=torch.float32, device=o_sparse_probe.device)
    _lib.call("bsa_probe_fit", B, Hq, Hkv, D, _ptr(o_sparse_probe), _ptr(o_dense_probe), _ptr(weights), M, nl,
              float(lam), int(rank), _ptr(A), _ptr(c), _stream())
    return A, c


def probe_apply(o: torch.Tensor, A: torch.Tensor, c: torch.Tensor) -> torch.Tensor:
    """o <- o + o A + c for every row, in place (bsa_probe_apply)."""
    _check_cuda(o, A, c)
    B, Hq, S, D = o.shape
    _lib.call("bsa_probe_apply", B, Hq, S, D, _dtype_code(o), _ptr(o), _ptr(A), _ptr(c), _stream())
    return o


# ----------------------------------------------------------------- head-wise mask reuse

def pooled_qk(q: torch.Tensor, k: torch.Tensor, Hm: Optional[int] = None,
              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token means of Q and K per mask head, float32 [B, Hm, D] each (bsa_pooled_qk).
    Hm defaults to the number of query heads."""
    _check_cuda(q, k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k shapes/dtypes do not match")
    Hm = Hq if Hm is None else int(Hm)
    qbar = torch.empty(B, Hm, D, dtype=torch.float32, device=q.device)
    kbar = torch.empty_like(qbar)
    nbytes = _lib.size_query("bsa_pooled_qk_workspace_size", B, Hq, Hkv, S, D)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    _lib.call("bsa_pooled_qk", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(k), Hm, _ptr(qbar), _ptr(kbar),
              _ptr(workspace), workspace.numel(), _stream())
    return qbar, kbar


def mask_reuse_decide(qbar: torch.Tensor, kbar: torch.Tensor, anchor_q: Optional[torch.Tensor],
                      anchor_k: Optional[torch.Tensor], delta: float, relative: bool = False,
                      gate: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Drift from the anchors and the refresh flags (uint8 [B, Hm]) with the optional layer
    gate (bsa_mask_reuse_decide).  anchor_q None: the first call, every head refreshes."""
    _check_cuda(qbar, kbar, anchor_q, anchor_k)
    B, Hm, D = qbar.shape
    have = anchor_q is not None
    if have and (anchor_k is None or anchor_q.shape != qbar.shape or anchor_k.shape != qbar.shape):
        raise ValueError("anchors must match the summaries")
    drift = torch.empty(B, Hm, dtype=torch.float32, device=qbar.device)
    refresh = torch.empty(B, Hm, dtype=torch.uint8, device=qbar.device)
    _lib.call("bsa_mask_reuse_decide", B, Hm, D, _ptr(qbar), _ptr(kbar), _ptr(anchor_q), _ptr(anchor_k), int(have),
              float(delta), int(relative), int(gate), _ptr(drift), _ptr(refresh), _stream())
    return drift, refresh


def mask_reuse_update(refresh: torch.Tensor, qbar: torch.Tensor, kbar: torch.Tensor, new_mask: Optional[BlockMask],
                      mask: Optional[BlockMask], anchor_q: torch.Tensor, anchor_k: torch.Tensor) -> None:
    """Refreshed heads take the new mask rows and move their anchors (bsa_mask_reuse_update)."""
    _check_cuda(refresh, qbar, kbar, anchor_q, anchor_k)
    B, Hm, D = qbar.shape
    if new_mask is not None:
        _, _, Cq, Ck = new_mask.keep.shape
        if mask is None or mask.keep.shape != new_mask.keep.shape:
            raise ValueError("the cached mask must match the new mask")
        args = (_ptr(new_mask.keep), _ptr(new_mask.kv_count), _ptr(new_mask.kv_idx), _ptr(mask.keep),
                _ptr(mask.kv_count), _ptr(mask.kv_idx))
    else:
        Cq = Ck = 1
        args = (None, None, None, None, None, None)
    _lib.call("bsa_mask_reuse_update", B, Hm, Cq, Ck, D, _ptr(refresh), _ptr(qbar), _ptr(kbar), *args, _ptr(anchor_q),
              _ptr(anchor_k), _stream())


class HeadMaskCache:
    """Per-head block masks and their anchors on the device, used in two phases per step
    ("Dynamic block masks and head-wise mask reuse", sections "HEART -- head-wise temporal
    mask reuse", "What mlx-arsenal ships" and "Recipe"):

        refresh = cache.should_refresh(q, k)          # uint8 [B, Hm] on the device
        scores = antidiagonal_block_scores(q, k, heads=refresh, out=...)   # refreshed heads only
        mask = cache.update(top_p_block_mask(scores, tau), refresh)

    One cache per layer (and per guidance branch); reset it when the token grid changes."""

    def __init__(self, delta: float, relative: bool = False, gate: bool = True, Hm: Optional[int] = None):
        self.delta, self.relative, self.gate, self.Hm = float(delta), bool(relative), bool(gate), Hm
        self.anchor_q: Optional[torch.Tensor] = None
        self.anchor_k: Optional[torch.Tensor] = None
        self.mask: Optional[BlockMask] = None
        self.drift: Optional[torch.Tensor] = None
        self._cur: Optional[Tuple[torch.Tensor, torch.Tensor]] = None

    def reset(self) -> None:
        self.anchor_q = self.anchor_k = self.mask = self.drift = self._cur = None

    def should_refresh(self, q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
        qbar, kbar = pooled_qk(q, k, self.Hm)
        self._cur = (qbar, kbar)
        self.drift, refresh = mask_reuse_decide(qbar, kbar, self.anchor_q, self.anchor_k, self.delta, self.relative,
                                                self.gate)
        return refresh

    def update(self, new_mask: BlockMask, refresh: torch.Tensor) -> BlockMask:
        if self._cur is None:
            raise RuntimeError("update() needs a preceding should_refresh()")
        qbar, kbar = self._cur
        if self.mask is None:  # first step: every head refreshed
            self.mask = BlockMask(new_mask.keep.clone(), new_mask.kv_count.clone(), new_mask.kv_idx.clone())
            self.anchor_q, self.anchor_k = qbar.clone(), kbar.clone()
        else:
            mask_reuse_update(refresh, qbar, kbar, new_mask, self.mask, self.anchor_q, self.anchor_k)
        self._cur = None
        return self.mask


# ----------------------------------------------------------------- response-coupled partitioning

def response_partition(q: torch.Tensor, k: torch.Tensor, Cq: int, Ck: int, scale: Optional[float] = None,
                       rK: int = 48, rQ: int = 64, iters: int = 4, return_centres: bool = False,
                       workspace: Optional[torch.Tensor] = None):
    """Key and query groups of every (batch, K/V head) from the call's own responses
    (bsa_response_partition): returns (k_labels, q_labels), int32 [B, Hkv, S] each, and with
    return_centres also the final k-means centres [B, Hkv, Ck, 64] and [B, Hkv, Cq, 64]."""
    _check_cuda(q, k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k shapes/dtypes do not match")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kl = torch.empty(B, Hkv, S, dtype=torch.int32, device=q.device)
    ql = torch.empty_like(kl)
    kc = torch.empty(B, Hkv, Ck, 64, dtype=torch.float32, device=q.device) if return_centres else None
    qc = torch.empty(B, Hkv, Cq, 64, dtype=torch.float32, device=q.device) if return_centres else None
    nbytes = _lib.size_query("bsa_response_partition_workspace_size", B, Hkv, S, D, Cq, Ck)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _workspace(nbytes, q.device)
    _lib.call("bsa_response_partition", B, Hq, Hkv, S, D, _dtype_code(q), _ptr(q), _ptr(k), float(scale), int(rK),
              int(rQ), int(Cq), int(Ck), int(iters), _ptr(kl), _ptr(ql), _ptr(kc), _ptr(qc), _ptr(workspace),
              workspace.numel(), _stream())
    return (kl, ql, kc, qc) if return_centres else (kl, ql)


def kmeans(x: torch.Tensor, C: int, iters: int = 4, nf: Optional[int] = None):
    """Batched k-means of float32 points x [P, N, 64] (features past nf zero) into C centres
    (bsa_kmeans): returns (labels int32 [P, N], centres float32 [P, C, 64])."""
    _check_cuda(x)
    P, N, F = x.shape
    if F != 64 or x.dtype != torch.float32:
        raise ValueError("x must be float32 [P, N, 64]")
    labels = torch.empty(P, N, dtype=torch.int32, device=x.device)
    centres = torch.empty(P, C, 64, dtype=torch.float32, device=x.device)
    ws = _workspace(_lib.size_query("bsa_kmeans_workspace_size", P, N, C), x.device)
    _lib.call("bsa_kmeans", P, N, int(nf or 64), _ptr(x), int(C), int(iters), _ptr(labels), _ptr(centres), _ptr(ws),
              ws.numel(), _stream())
    return labels, centres


def select_probe_rows(labels: np.ndarray, C: int, M: int) -> Tuple[np.ndarray, np.ndarray]:
    """Host helper: probe rows and normalized weights (bsa_select_probe_rows)."""
    lab = np.ascontiguousarray(labels, dtype=np.int32)
    idx = np.empty(M, dtype=np.int32)
    w = np.empty(M, dtype=np.float32)
    _lib.call("bsa_select_probe_rows", lab.ctypes.data_as(ctypes.c_void_p), lab.size, C, M,
              idx.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p))
    return idx, w


def sliding_tile_block_mask(nT: int, nH: int, nW: int, tile=(1, 1, 1), window=(1, 1, 1)) -> np.ndarray:
    """Host helper: static sliding-tile keep bits uint8 [N, N] over the cells of a raster
    nT x nH x nW grid (bsa_sliding_tile_mask); with tile = (1, 1, 1) the cluster-level mask
    for tile_labels clusters.  Use mask_from_keep to hand it to the attention."""
    N = nT * nH * nW
    out = np.empty((N, N), dtype=np.uint8)
    _lib.call("bsa_sliding_tile_mask", nT, nH, nW, int(tile[0]), int(tile[1]), int(tile[2]), int(window[0]),
              int(window[1]), int(window[2]), out.ctypes.data_as(ctypes.c_void_p))
    return out


def tile_labels(T: int, H: int, W: int, tile, chunk: int = 0) -> np.ndarray:
    """Host helper: sliding-tile labels of a raster T x H x W grid (bsa_tile_labels)."""
    out = np.empty(T * H * W, dtype=np.int32)
    _lib.call("bsa_tile_labels", T, H, W, int(tile[0]), int(tile[1]), int(tile[2]), int(chunk),
              out.ctypes.data_as(ctypes.c_void_p))
    return out
