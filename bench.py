#!/usr/bin/env python3
"""Benchmark of the whole block-sparse attention path on one MI355X.

Workload: the Wan-shaped video case -- B=1, 40 heads, S=32760 tokens (a 21x30x52 latent
grid), D=128, bfloat16, 256 tile-major clusters of 128 tokens (the last holds 120) --
run through every stage of the path in one call: cluster layout, K/V packing with the
centroids, antidiagonal
block scores (block 128, stride 16), per-head top-p masks (tau per head from
{0.85, 0.90, 0.95}), 64 probe rows (dense and block-sparse), the ridge fit (lambda 0.1,
rank 16), and the compensated block-sparse attention whose epilogue applies the fitted
correction.  Inputs are seeded synthetic fields (synthetic.make_config(2)) resident in
HBM before timing starts.

Printed: one JSON line.  ``value`` is the executed-pair throughput of the whole call
(4*D flops per executed token pair: kept-block pairs plus the probe rows' dense pairs,
over the measured time per call); ``ms_per_step`` is the time per call.  ``roofline``
covers the dominant kernel (the sparse attention): its algorithmic flops (4*D per kept
token pair) over its average launch time, measured with events on the stream it runs on,
against the bf16 dense MFMA peak; ``traffic`` is the kernel's HBM bytes per launch from the
rocprofv3 counter summary in profiles/ when that summary was taken on the current kernel
sources (else null).  ``cpu_baseline`` is the float64 CPU oracle timed on a bounded sample
of the same workload (one head, a subset of query clusters).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --profile-kernels K   # for rocprofv3: K launches of each kernel alone,
                                          # then one plain copy of a known size
    python bench.py --summarize-profiles DIR  # write the profiles/ summaries from the csv
                                              # files of the PROFILE_COMMANDS runs in DIR
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/call + executed-pair TFLOP/s (% MFMA peak), S=32760 H=40 D=128 bf16"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PROBES, LAMBDA, RANK = 64, 0.1, 16
WORKLOAD = ("wan_video_21x30x52_S32760_H40_D128_bf16: scored top-p masks + compensated block-sparse "
            "attention + 64-probe ridge repair")
COPY_BYTES = 1 << 30  # the reference copy for scaling the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_kernel_wan_S32760_H40_D128_traffic.json")
KERNEL_SOURCES = ("attention.hip", "pack.hpp", "common.hpp")
ATTN_KERNEL = "sparse_attn_kernel"
# The rocprofv3 runs behind the profiles/ summaries, from the repository root; each writes
# <name>_*.csv into the directory given after -d, which --summarize-profiles then reads.
PROFILE_COMMANDS = {
    "trace": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $R/gpurun_out/prof -o trace -- python3 $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline",
    "fetch": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
             "-d $R/gpurun_out/prof -o fetch -- python3 $R/bench.py --profile-kernels 3 --no-cpu-baseline",
    "write": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
             "-d $R/gpurun_out/prof -o write -- python3 $R/bench.py --profile-kernels 3 --no-cpu-baseline",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_antidiagonal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it was taken on
    the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _short_kernel(name: str) -> str:
    name = name.replace("void ", "").replace("bsa::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:  # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def _counter_per_dispatch(path: str):
    """{kernel: [counter value per dispatch]} from a rocprofv3 counter_collection csv."""
    import csv

    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            per.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def summarize_profiles(d: str) -> int:
    """Write the kernel-trace table, the HBM counter table and the attention kernel's traffic
    record (profiles/) from the csv files of the PROFILE_COMMANDS runs in directory d."""
    import csv

    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    stem = "wan_S32760_H40_D128"
    stats = os.path.join(d, "trace_kernel_stats.csv")
    if os.path.exists(stats):
        rows = list(csv.DictReader(open(stats)))
        lines = [f"# Kernel trace: whole path, video workload (B=1, H=40, S=32760, D=128, bf16)", "",
                 "Command (from the repository root, on one MI355X):", "", "```", PROFILE_COMMANDS["trace"], "```",
                 "", "7 calls per path kernel = 2 warmup + 5 timed path calls.  The other dispatches come from "
                 "the same run's mask-reuse, sliding-tile and error-aware-routing measurements (the "
                 "`bfloat16`-output attention kernel runs the sliding-tile and the routed masks).  "
                 "Durations in microseconds.", "",
                 "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
        for r in rows:
            lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                         f"{float(r['Percentage']):.2f} |")
        with open(os.path.join(out_dir, f"path_kernels_{stem}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    fetch = os.path.join(d, "fetch_counter_collection.csv")
    write = os.path.join(d, "write_counter_collection.csv")
    if not (os.path.exists(fetch) and os.path.exists(write)):
        return 0
    fe, wr = _counter_per_dispatch(fetch), _counter_per_dispatch(write)
    copy = "__amd_rocclr_copyBuffer"
    # The plain copy moves COPY_BYTES each way, possibly over several dispatches.
    fetch_scale = COPY_BYTES / (sum(fe[copy]) * 1024.0)
    write_scale = COPY_BYTES / (sum(wr[copy]) * 1024.0)
    lines = ["# HBM byte counters per dispatch, video workload (B=1, H=40, S=32760, D=128, bf16)", "",
             "Commands (from the repository root, on one MI355X), one counter per run:", "", "```",
             PROFILE_COMMANDS["fetch"], PROFILE_COMMANDS["write"], "```", "",
             f"Each run ends with one plain device copy of {COPY_BYTES} bytes.  Its counters, summed over its "
             f"dispatches, read {sum(fe[copy]):.0f} KiB (FETCH_SIZE) and {sum(wr[copy]):.0f} KiB (WRITE_SIZE), "
             f"so the counters below are scaled by {fetch_scale:.3f} and {write_scale:.3f} to bytes.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB |",
             "|---|---:|---:|---:|---:|---:|"]
    traffic = None
    for k in fe:
        if k == copy or k not in wr:
            continue
        f_kib = sum(fe[k]) / len(fe[k])
        w_kib = sum(wr[k]) / len(wr[k])
        rd, wt = f_kib * 1024 * fetch_scale, w_kib * 1024 * write_scale
        lines.append(f"| `{k}` | {len(fe[k])} | {f_kib:.0f} | {w_kib:.0f} | {rd / 1e9:.3f} | {wt / 1e9:.3f} |")
        if k.startswith(ATTN_KERNEL) and (traffic is None or rd + wt > traffic["bytes_per_launch"]):
            traffic = {"kernel": k, "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": fetch_scale,
                       "write_scale": write_scale, "read_bytes": rd, "write_bytes": wt,
                       "bytes_per_launch": rd + wt, "source_sha256": kernel_source_hash(),
                       "commands": [PROFILE_COMMANDS["fetch"], PROFILE_COMMANDS["write"]]}
    with open(os.path.join(out_dir, f"hbm_counters_{stem}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if traffic is not None:
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(traffic, f, indent=1)
            f.write("\n")
    return 0


def executed_pairs(res, cfg):
    """Kept token pairs per call (sum over heads and query clusters of n_a times the kept key
    tokens) -- a measurement of the mask, computed with torch on the GPU."""
    import torch

    keep = res.mask.keep.to(torch.float64)  # [B, Hm, Cq, Ck]
    n = res.layout.counts.to(torch.float64)  # [C]
    kept_keys = keep @ n  # [B, Hm, Cq]
    per_mask_head = (kept_keys * n).sum(dim=-1)  # [B, Hm]
    Hm = keep.shape[1]
    heads_per_mask = cfg.Hq // Hm
    return float(per_mask_head.sum().item()) * heads_per_mask


def cpu_baseline(wl, seconds_hint=20.0):
    """The float64 oracle on a bounded sample: head 0, its scores and mask, the attention
    rows of every 2nd query cluster, the 64 probe rows and the fit."""
    from oracle import pipeline

    try:
        import threadpoolctl

        threads = max((d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    clusters = list(range(0, wl.C, 2))
    rows = np.nonzero(np.isin(wl.labels, clusters))[0]
    t0 = time.perf_counter()
    keep = pipeline.head_mask(wl, 0, 0)
    res = pipeline.run_head(wl, 0, 0, rows=rows, keep=keep)
    elapsed = time.perf_counter() - t0
    counts = np.bincount(wl.labels, minlength=wl.C)
    kept_keys = keep.astype(np.float64) @ counts
    pairs = float(kept_keys[wl.labels[rows]].sum()) + wl.probes * wl.S
    del res
    return {
        "value": 4 * wl.D * pairs / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"head 0 of {wl.Hq}: scores + top-p mask, compensated attention for {rows.size} rows "
                   f"({len(clusters)} of {wl.C} query clusters), {wl.probes} dense probe rows, ridge fit; "
                   f"{elapsed:.1f} s"),
        "seconds": elapsed,
    }


def measure_reuse(bsa, cfg, q, k, res, reps=10):
    """Head-wise mask reuse on the same inputs, timed with events on the current stream:
    the pooled Q/K pass (reads Q and K once), the drift/gate decision, and one cache step
    (summary + decision + predictor for the refreshed heads + top-p + cache update) when
    every head rebuilds its mask (a new cache) and when no head does (the same Q and K again,
    drift 0)."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api

    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    score_scale = cfg.score_scale or 1.0 / math.sqrt(cfg.D)
    Hs = cfg.Hkv if cfg.pool_gqa else cfg.Hq
    nb = -(-cfg.S // cfg.block)
    scores = torch.empty(cfg.B, Hs, nb, nb, dtype=torch.float32, device=q.device)
    ws = torch.empty(bsa._lib.size_query("bsa_antidiag_scores_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D,
                                         cfg.block, cfg.stride), dtype=torch.uint8, device=q.device)
    tau = torch.as_tensor(np.asarray(cfg.tau, dtype=np.float32).reshape(-1)).to(q.device)
    qbar, kbar = api.pooled_qk(q, k, Hs)
    pooled_ms = timed(lambda: api.pooled_qk(q, k, Hs))
    anchors = (qbar.clone(), kbar.clone())
    decide_ms = timed(lambda: api.mask_reuse_decide(qbar, kbar, *anchors, 1.0))

    def step(cache):
        refresh = cache.should_refresh(q, k)
        api.antidiagonal_block_scores(q, k, res.layout, cfg.block, cfg.stride, score_scale, cfg.pool_gqa,
                                      workspace=ws, heads=refresh, out=scores)
        return cache.update(api.top_p_block_mask(scores, tau), refresh)

    def rebuild():
        step(api.HeadMaskCache(delta=1.0))

    warm = api.HeadMaskCache(delta=1.0)
    step(warm)
    rebuild_ms = timed(rebuild)
    reuse_ms = timed(lambda: step(warm))  # same Q and K: drift 0, every head keeps its mask
    torch.cuda.synchronize()
    qk_bytes = cfg.B * (cfg.Hq + cfg.Hkv) * cfg.S * cfg.D * q.element_size()
    gbs = qk_bytes / (pooled_ms * 1e-3) / 1e9
    return {
        "pooled_qk_ms": round(pooled_ms, 4),
        "pooled_qk_GBps": round(gbs, 1),
        "pooled_qk_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "decide_ms": round(decide_ms, 4),
        "step_all_rebuild_ms": round(rebuild_ms, 4),
        "step_all_reuse_ms": round(reuse_ms, 4),
    }


STA_TILE = (2, 8, 8)  # 128-token tiles of the 21 x 30 x 52 latent grid (edge tiles partial)
STA_WINDOW = (7, 3, 3)  # tiles: 63 of the 11 x 4 x 7 = 308 tiles per row


def measure_sliding_tile(bsa, cfg, wl, q, k, v, reps=5):
    """The compensated attention on a static sliding-tile mask over the same Q, K, V: tile
    labels as the clusters and the tile-level mask from the host helper, timed with events on
    the current stream (the kernel's second workload: a static mask instead of a scored one)."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api

    T, H, W = wl.grid
    labels = api.tile_labels(T, H, W, STA_TILE)
    C = int(labels.max()) + 1
    nt, nh, nw = (-(-T // STA_TILE[0]), -(-H // STA_TILE[1]), -(-W // STA_TILE[2]))
    keep_tile = api.sliding_tile_block_mask(nt, nh, nw, (1, 1, 1), STA_WINDOW)
    layout = api.cluster_layout(torch.from_numpy(labels).to(q.device), C)
    kv = api.kv_pack(k, v, layout)
    keep = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(keep_tile, (cfg.B, cfg.Hkv, C, C)))).to(q.device)
    mask = api.mask_from_keep(keep)
    ws = api.attention_workspace(q, kv, layout, mask)
    out = torch.empty_like(q)

    def run():
        api.block_sparse_attention(q, kv, layout, mask, True, cfg.scale, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = np.bincount(labels, minlength=C).astype(np.float64)
    pairs = float((keep_tile.astype(np.float64) @ n) @ n) * cfg.B * cfg.Hq
    tflops = 4 * cfg.D * pairs / (ms * 1e-3) / 1e12
    return {
        "tile": list(STA_TILE), "window_tiles": list(STA_WINDOW), "clusters": C,
        "density": round(pairs / (cfg.B * cfg.Hq * float(cfg.S) ** 2), 4),
        "attention_ms": round(ms, 4), "executed_pair_TFLOPs": round(tflops, 2),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
    }


def measure_routing(bsa, cfg, q, k, v, res, density, reps=5):
    """Error-aware routing on the same Q, K, V and clusters as the path: the query-centroid
    probes, the per-block errors (a dense pass of the Cq probes per head, then the per-cluster
    sums) and the routes under a key budget equal to the scored masks' density, then the
    compensated attention on the routed masks.  Each stage is timed alone with events on the
    current stream."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api

    layout = res.layout
    kv = api.kv_pack(k, v, layout)
    budget = int(round(density * cfg.S))
    ws = torch.empty(_lib_size("bsa_block_error_workspace_size", cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D, layout.C,
                               layout.C), dtype=torch.uint8, device=q.device)
    qbar = api.query_centroids(q, layout)
    err = api.block_error(qbar, kv, cfg.scale, workspace=ws)
    mask = api.error_route(err, layout, budget)
    aws = api.attention_workspace(q, kv, layout, mask)
    out = torch.empty_like(q)
    stages = {
        "probes": lambda: api.query_centroids(q, layout),
        "block_error": lambda: api.block_error(qbar, kv, cfg.scale, workspace=ws),
        "route": lambda: api.error_route(err, layout, budget),
        "attention": lambda: api.block_sparse_attention(q, kv, layout, mask, True, cfg.scale, out=out, workspace=aws),
    }
    stream = torch.cuda.current_stream()
    ms = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    n = layout.counts.double()
    pairs = float(((mask.keep.double() @ n) * n).sum()) * (cfg.Hq // mask.keep.shape[1])
    # Two passes of the Cq probes over every key: 4 D flops per (probe, key) pair each.
    err_flops = 2 * 4 * cfg.D * layout.C * cfg.S * cfg.B * cfg.Hq
    att_tflops = 4 * cfg.D * pairs / (ms["attention"] * 1e-3) / 1e12
    return {
        "budget_tokens": budget, "density": round(pairs / (cfg.B * cfg.Hq * float(cfg.S) ** 2), 4),
        "probes_ms": round(ms["probes"], 4), "block_error_ms": round(ms["block_error"], 4),
        "route_ms": round(ms["route"], 4),
        "block_error_TFLOPs": round(err_flops / (ms["block_error"] * 1e-3) / 1e12, 2),
        "block_error_mfma_frac": round(err_flops / (ms["block_error"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "attention_ms": round(ms["attention"], 4), "attention_executed_pair_TFLOPs": round(att_tflops, 2),
    }


def _lib_size(name, *args):
    from block_sparse_attention_antidiagonal_amd import _lib
    return _lib.size_query(name, *args)


def profile_kernels(bsa, path, cfg, q, k, v, reps):
    """One path call, then `reps` launches of the pack, the scores and the attention alone,
    then one plain device copy of COPY_BYTES (reads and writes that many bytes)."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api

    res = path(q, k, v)
    torch.cuda.synchronize()
    kv = api.kv_pack(k, v, res.layout)
    ws = api.attention_workspace(q, kv, res.layout, res.mask)
    o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    for i in range(reps):
        api.kv_pack(k, v, res.layout, kv.buffer)
        torch.cuda.synchronize()
        print(f"[profile] pack {i}", flush=True)
    for i in range(reps):
        api.antidiagonal_block_scores(q, k, res.layout, cfg.block, cfg.stride,
                                      cfg.score_scale or 1.0 / math.sqrt(cfg.D), cfg.pool_gqa)
        torch.cuda.synchronize()
        print(f"[profile] scores {i}", flush=True)
    for i in range(reps):
        api.block_sparse_attention(q, kv, res.layout, res.mask, cfg.compensate, cfg.scale, out=o32, out_f32=True,
                                   workspace=ws)
        torch.cuda.synchronize()
        print(f"[profile] attention {i}", flush=True)
    for i in range(reps):
        api.pooled_qk(q, k)
        torch.cuda.synchronize()
        print(f"[profile] pooled_qk {i}", flush=True)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=q.device).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[profile] copy {COPY_BYTES} bytes", flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the K/V packing and probe rows on the caller's stream too")
    ap.add_argument("--profile-kernels", type=int, default=0, metavar="K",
                    help="launch each kernel K times on its own, then one plain copy (for rocprofv3)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 csv files in DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X (asked for --gpus {args.gpus}). "
              "Heads and K/V groups are independent, so a multi-GPU run would shard them without exchange.",
              file=sys.stderr)
        return 2

    import torch

    import block_sparse_attention_antidiagonal_amd as bsa
    from synthetic import make_config

    print("[bench] generating inputs", file=sys.stderr, flush=True)
    wl = make_config(2)
    wl.probes, wl.lam, wl.rank = PROBES, LAMBDA, RANK
    cfg = bsa.PathConfig.from_workload(wl)
    cfg.overlap = not args.no_overlap
    path = bsa.SparseAttentionPath(cfg)
    q = torch.from_numpy(wl.q).to(torch.bfloat16).cuda()
    k = torch.from_numpy(wl.k).to(torch.bfloat16).cuda()
    v = torch.from_numpy(wl.v).to(torch.bfloat16).cuda()
    torch.cuda.synchronize()

    if args.profile_kernels:
        return profile_kernels(bsa, path, cfg, q, k, v, args.profile_kernels)

    print("[bench] warmup", file=sys.stderr, flush=True)
    res = None
    for _ in range(args.warmup):
        res = path(q, k, v)
    torch.cuda.synchronize()
    if res is None:
        res = path(q, k, v)
        torch.cuda.synchronize()
    pairs = executed_pairs(res, cfg)
    density = pairs / (cfg.B * cfg.Hq * float(cfg.S) ** 2)
    probe_pairs = float(cfg.B * cfg.Hq * PROBES * cfg.S)

    print("[bench] timing", file=sys.stderr, flush=True)
    marks = []  # per step: list of (stage, event)

    def recorder(step_marks):
        last = {}  # stream -> its latest event; a stage spans from there to its own mark

        def mark(name):
            stream = torch.cuda.current_stream()
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            if stream.cuda_stream in last:
                step_marks.append((name, last[stream.cuda_stream], ev))
            last[stream.cuda_stream] = ev
        return mark

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sm = []
        path(q, k, v, mark=recorder(sm))
        marks.append(sm)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    stages = {}
    for sm in marks:
        for name, e0, e1 in sm:
            stages.setdefault(name, []).append(e0.elapsed_time(e1))
    stages_ms = {name: float(np.mean(v)) for name, v in stages.items()}
    attn_ms = stages_ms["attention"]

    D, S, H = cfg.D, cfg.S, cfg.Hq
    value = 4 * D * (pairs + probe_pairs) / (ms_per_step * 1e-3) / 1e12
    attn_flops = 4 * D * pairs
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    kv_bytes = 2 * cfg.B * cfg.Hkv * S * D * 2
    B_H_S_D = cfg.B * cfg.Hq * S * D
    traffic = measured_traffic()
    qk_bytes = cfg.B * (cfg.Hq + cfg.Hkv) * S * D * 2
    score_flops = 2 * cfg.B * cfg.Hq * (math.ceil(S / 128) * 128) ** 2 * D / 16

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD,
            "B": cfg.B, "H": H, "S": S, "D": D, "block": 128, "stride": 16,
            "tau": "per head from {0.85, 0.90, 0.95}", "density": round(density, 4),
            "probes": PROBES, "lambda": LAMBDA, "rank": RANK, "compensation": True,
        },
        "ms_per_call": round(ms_per_step, 4),
        "executed_pairs": pairs + probe_pairs,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "sparse_attn_kernel (compensated, float32 rows)",
            "algorithmic_tflop_per_launch": attn_flops / 1e12,
            "avg_launch_ms": round(attn_ms, 4),
        },
        "stages_ms": {kk: round(vv, 4) for kk, vv in stages_ms.items()},
        "stage_rates": {
            # the pack reads K and V once and writes them once as tiles
            "pack_GBps": round(2 * kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9, 1),
            "pack_hbm_frac": round(2 * kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            # the correction reads the float32 rows and writes the bfloat16 output once
            "correct_GBps": round(3 * B_H_S_D * 2 / (stages_ms["correct"] * 1e-3) / 1e9, 1),
            "correct_hbm_frac": round(3 * B_H_S_D * 2 / (stages_ms["correct"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_GBps": round(qk_bytes / (stages_ms["scores"] * 1e-3) / 1e9, 1),
            "scores_hbm_frac": round(qk_bytes / (stages_ms["scores"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_TFLOPs": round(score_flops / (stages_ms["scores"] * 1e-3) / 1e12, 2),
            "scores_mfma_frac": round(score_flops / (stages_ms["scores"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
    }
    print("[bench] mask reuse", file=sys.stderr, flush=True)
    line["mask_reuse"] = measure_reuse(bsa, cfg, q, k, res)
    print("[bench] sliding-tile mask", file=sys.stderr, flush=True)
    line["sliding_tile_attention"] = measure_sliding_tile(bsa, cfg, wl, q, k, v)
    print("[bench] error-aware routing", file=sys.stderr, flush=True)
    line["error_aware_routing"] = measure_routing(bsa, cfg, q, k, v, res, line["config"]["density"])
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(wl)
        cb["value"] = round(cb["value"], 6)
        cb.pop("seconds", None)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
