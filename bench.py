#!/usr/bin/env python3
"""Benchmark of the whole block-sparse attention path on one MI355X.

Headline workload: the Wan-shaped video case -- B=1, 40 heads, S=32760 tokens (a 21x30x52
latent grid), D=128, bfloat16, 256 tile-major clusters of 128 tokens (the last holds 120)
-- run through every stage of the path in one call: cluster layout, K/V packing with the
centroids, antidiagonal block scores (block 128, stride 16), per-head top-p masks (tau per
head from {0.85, 0.90, 0.95}) and the compensated block-sparse attention.  Inputs are seeded
synthetic fields (synthetic.make_config(2)) resident in HBM before timing starts.

Beside it, the two repair workloads are timed the same way (``repair_workloads``): the same
inputs run as hard-drop attention with 64-probe ridge repair, and the grouped-query case
(B=2, 40 query heads on 8 K/V heads, pooled masks, compensation and repair).

Printed: one JSON line.  ``value`` is the executed-pair throughput of the whole call
(4*D flops per kept token pair over the measured time per call); ``ms_per_step`` is the
time per call.  ``roofline`` covers the dominant kernel (the sparse attention): its
algorithmic flops (4*D per kept token pair) over its average launch time, measured with
events on the stream it runs on, against the bf16 dense MFMA peak; ``traffic`` is the
kernel's HBM bytes per launch from the rocprofv3 counter summary in profiles/ when that
summary was taken on the current kernel sources (else null).  ``cpu_baseline`` is the
float64 CPU oracle timed on a bounded sample of the same workload (one head, a subset of
query clusters).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--path-only]
    python bench.py --profile-kernels K   # for rocprofv3: K launches of each kernel alone,
                                          # then one plain copy of a known size
    python bench.py --summarize-profiles DIR  # write the profiles/ summaries from the csv
                                              # files of the PROFILE_COMMANDS runs in DIR
"""

from __future__ import annotations

import argparse
import dataclasses
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
WORKLOAD = ("wan_video_21x30x52_S32760_H40_D128_bf16: antidiagonal scores + per-head top-p masks + "
            "compensated block-sparse attention")
COPY_BYTES = 1 << 30  # the reference copy for scaling the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_kernel_wan_S32760_H40_D128_traffic.json")
KERNEL_SOURCES = ("attention.hip", "pack.hpp", "common.hpp")
ATTN_KERNEL = "sparse_attn_kernel"
TRACE_STEPS, TRACE_WARMUP = 5, 2  # the path calls of the "trace" command below
# The rocprofv3 runs behind the profiles/ summaries, from the repository root; each writes
# <name>_*.csv into the directory given after -d, which --summarize-profiles then reads.
PROFILE_COMMANDS = {
    "trace": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $R/gpurun_out/prof -o trace -- python3 $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline "
             "--path-only > $R/gpurun_out/prof/trace_bench.json",
    "fetch": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
             "-d $R/gpurun_out/prof -o fetch -- python3 $R/bench.py --profile-kernels 3 --no-cpu-baseline",
    "write": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
             "-d $R/gpurun_out/prof -o write -- python3 $R/bench.py --profile-kernels 3 --no-cpu-baseline",
    # MFMA, VALU and LDS activity, then the L2 hit rate, of the same launches
    "sq": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA "
          "SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVES GRBM_GUI_ACTIVE "
          "--output-format csv -d $R/gpurun_out/prof -o sq -- python3 $R/bench.py --profile-kernels 3 "
          "--no-cpu-baseline",
    "l2": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv "
          "-d $R/gpurun_out/prof -o l2 -- python3 $R/bench.py --profile-kernels 3 --no-cpu-baseline",
    # the grouped-query workload's attention alone: HBM bytes, then L2 hits (its five query
    # heads of a group share their K/V tiles through L2)
    "gqa_fetch": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
                 "-d $R/gpurun_out/prof -o gqa_fetch -- python3 $R/bench.py --profile-gqa 3",
    "gqa_l2": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv "
              "-d $R/gpurun_out/prof -o gqa_l2 -- python3 $R/bench.py --profile-gqa 3",
    # where the waves' time goes: waiting to issue, waiting on memory/LDS, VALU beside MFMA
    "issue": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY "
             "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
             "SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE --output-format csv -d $R/gpurun_out/prof -o issue -- python3 "
             "$R/bench.py --profile-kernels 3 --no-cpu-baseline",
    # LDS and vector-memory occupancy: LDS busy cycles and bytes read/written by LDS
    # instructions, the address (TA) and data (TD) units of the vector memory path, and the
    # cycles their queues were full
    "lds": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
           "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_INSTS_LDS_STORE_BANDWIDTH SQ_LDS_DATA_FIFO_FULL SQ_VMEM_TA_ADDR_FIFO_FULL "
           "SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE TA_BUSY_avr TA_BUFFER_TOTAL_CYCLES_sum TD_TD_BUSY_sum "
           "--output-format csv -d $R/gpurun_out/prof -o lds -- python3 $R/bench.py --profile-kernels 3 "
           "--no-cpu-baseline",
    # the partitioned (SparsePR) call alone
    "trace_partitioned": "R=$PWD; cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format "
                         "csv -d $R/gpurun_out/prof -o trace_partitioned -- python3 $R/bench.py --steps 5 "
                         "--warmup 2 --partitioned-only",
}
SIMDS, NOMINAL_GHZ, XCDS = 1024, 2.4, 8  # MI355X: 256 CUs x 4 SIMDs, peak engine clock, XCDs


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


def _summarize_trace(trace: str, command: str, out_path: str, title: str) -> None:
    """Kernel-trace table of a run of TRACE_STEPS + TRACE_WARMUP calls (warm-up launches dropped)."""
    import csv

    if not os.path.exists(trace):
        return
    calls, warm = TRACE_STEPS + TRACE_WARMUP, TRACE_WARMUP
    per = {}
    with open(trace) as f:
        for r in csv.DictReader(f):
            per.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = [f"# Kernel trace: {title}", "", "Command (from the repository root, on one MI355X):", "", "```",
             PROFILE_COMMANDS[command], "```", "",
             f"The run makes {calls} calls: {warm} warm-up calls, then the {TRACE_STEPS} timed calls.  Kernels "
             f"launched a whole number of times per call are summarized over the timed calls' launches; durations "
             f"in microseconds.", "",
             "| kernel | launches per call | timed launches | avg us | min us | max us | us per call |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    total = 0.0
    for k, ds in sorted(per.items(), key=lambda kv: -sum(x for _, x in kv[1])):
        ds.sort()
        if len(ds) % calls:
            lines.append(f"| `{k}` | ? | {len(ds)} (all) | {np.mean([x for _, x in ds]):.1f} | "
                         f"{min(x for _, x in ds):.1f} | {max(x for _, x in ds):.1f} | |")
            continue
        m = len(ds) // calls
        timed = [x for _, x in ds[warm * m:]]
        total += sum(timed) / TRACE_STEPS
        lines.append(f"| `{k}` | {m} | {len(timed)} | {np.mean(timed):.1f} | {min(timed):.1f} | {max(timed):.1f} | "
                     f"{sum(timed) / TRACE_STEPS:.1f} |")
    lines += ["", f"Kernel time per timed call: {total:.1f} us."]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counters_by_dispatch(path: str):
    """{kernel: [{counter: value, "dur_ns": ...} per dispatch]} from a counter_collection csv."""
    import csv

    disp = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], _short_kernel(r["Kernel_Name"]))
            e = disp.setdefault(key, {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
    per = {}
    for (_, k), e in sorted(disp.items(), key=lambda kv: int(kv[0][0])):
        per.setdefault(k, []).append(e)
    return per


def _summarize_counters(d: str, out_path: str) -> None:
    """MFMA busy, instruction mix, LDS bank conflicts and L2 hit rate per kernel, from the "sq"
    and "l2" runs (dispatches shorter than 20 us, such as the path's empty general-queue
    attention launch, are left out)."""
    sq_csv, l2_csv = os.path.join(d, "sq_counter_collection.csv"), os.path.join(d, "l2_counter_collection.csv")
    if not (os.path.exists(sq_csv) and os.path.exists(l2_csv)):
        return
    sq, l2 = _counters_by_dispatch(sq_csv), _counters_by_dispatch(l2_csv)
    lines = ["# SQ and L2 counters per kernel, video workload (B=1, H=40, S=32760, D=128, bf16)", "",
             "Commands (from the repository root, on one MI355X), one counter set per run:", "", "```",
             PROFILE_COMMANDS["sq"], PROFILE_COMMANDS["l2"], "```", "",
             "Per kernel, the mean over its dispatches of at least 20 us.  MFMA busy is "
             "SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles of the dispatch, counted two ways: at the nominal "
             f"{NOMINAL_GHZ} GHz (duration x {NOMINAL_GHZ} GHz x {SIMDS} SIMDs; comparable with the fraction of "
             f"the {PEAK_BF16_TFLOPS:.0f} TFLOP/s peak) and at the clock the counters saw (GRBM_GUI_ACTIVE, "
             f"summed over the {XCDS} XCDs, divided by {XCDS}: the busy share of the cycles that elapsed).  "
             "LDS conflicts are SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE; L2 hits are TCC_HIT over "
             "TCC_HIT + TCC_MISS.", "",
             "| kernel | dispatches | us | clock GHz | MFMA busy @2.4 GHz | MFMA busy @seen clock | MFMA insts | "
             "VALU insts | LDS insts | LDS conflict | L2 hit |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    rows = []
    for k, ds in sq.items():
        ds = [e for e in ds if e["dur_ns"] >= 20000]
        if not ds or k.startswith("__amd"):
            continue
        mean = lambda key: float(np.mean([e.get(key, 0.0) for e in ds]))
        dur = mean("dur_ns")
        busy, grbm = mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE")
        clk = grbm / XCDS / dur if dur > 0 else 0.0
        lds_act = mean("SQ_LDS_IDX_ACTIVE")
        conf = mean("SQ_LDS_BANK_CONFLICT") / lds_act if lds_act > 0 else 0.0
        l2d = [e for e in l2.get(k, []) if e["dur_ns"] >= 20000]
        hit = float(np.mean([e.get("TCC_HIT_sum", 0.0) for e in l2d])) if l2d else 0.0
        miss = float(np.mean([e.get("TCC_MISS_sum", 0.0) for e in l2d])) if l2d else 0.0
        rows.append((dur, f"| `{k}` | {len(ds)} | {dur / 1e3:.1f} | {clk:.2f} | "
                          f"{100 * busy / (dur * NOMINAL_GHZ * SIMDS):.1f}% | "
                          f"{100 * busy / (grbm / XCDS * SIMDS) if grbm > 0 else 0.0:.1f}% | {mean('SQ_INSTS_MFMA'):.3g} | "
                          f"{mean('SQ_INSTS_VALU'):.3g} | {mean('SQ_INSTS_LDS'):.3g} | {100 * conf:.1f}% | "
                          f"{100 * hit / (hit + miss) if hit + miss > 0 else 0.0:.1f}% |"))
    lines += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    issue_csv = os.path.join(d, "issue_counter_collection.csv")
    if os.path.exists(issue_csv):
        iss = _counters_by_dispatch(issue_csv)
        lines += ["", "## Issue and wait counters", "", "```", PROFILE_COMMANDS["issue"], "```", "",
                  "Per kernel, the mean over its dispatches of at least 20 us.  Wave shares are over the waves' "
                  "resident cycles (SQ_WAVE_CYCLES): waiting to issue (SQ_WAIT_INST_ANY: an instruction is ready "
                  "but its unit is taken, e.g. by the other wave's MFMAs), waiting on a counter or barrier "
                  "(SQ_WAIT_ANY), issuing VALU (SQ_ACTIVE_INST_VALU) and LDS (SQ_ACTIVE_INST_LDS) work; per SIMD "
                  "over the cycles that elapsed at the seen clock: MFMA busy and cycles in which a VALU "
                  "instruction issued while the MFMA unit was busy (SQ_VALU_MFMA_COEXEC_CYCLES).", "",
                  "| kernel | us | clock GHz | waves per SIMD | wait to issue | wait on counter | VALU issue | "
                  "LDS issue | MFMA busy | VALU beside MFMA |",
                  "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        rows = []
        for k, ds in iss.items():
            ds = [e for e in ds if e["dur_ns"] >= 20000]
            if not ds or k.startswith("__amd"):
                continue
            mean = lambda key: float(np.mean([e.get(key, 0.0) for e in ds]))
            dur, grbm = mean("dur_ns"), mean("GRBM_GUI_ACTIVE")
            elapsed = grbm / XCDS  # cycles at the seen clock
            wave = 4.0 * mean("SQ_WAVE_CYCLES")  # the SQ wave counters count quad-cycles
            if elapsed <= 0 or wave <= 0:
                continue
            share = lambda key: 100.0 * 4.0 * mean(key) / wave
            rows.append((dur, f"| `{k}` | {dur / 1e3:.1f} | {elapsed / dur:.2f} | {wave / SIMDS / elapsed:.2f} | "
                              f"{share('SQ_WAIT_INST_ANY'):.1f}% | {share('SQ_WAIT_ANY'):.1f}% | "
                              f"{share('SQ_ACTIVE_INST_VALU'):.1f}% | {share('SQ_ACTIVE_INST_LDS'):.1f}% | "
                              f"{100 * mean('SQ_VALU_MFMA_BUSY_CYCLES') / (SIMDS * elapsed):.1f}% | "
                              f"{100 * mean('SQ_VALU_MFMA_COEXEC_CYCLES') / (SIMDS * elapsed):.1f}% |"))
        lines += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    lines += _summarize_lds(d)
    lines += _summarize_gqa(d)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _summarize_lds(d: str) -> list:
    """LDS and vector-memory occupancy per kernel from the "lds" run: the share of elapsed CU
    cycles in which the LDS served indexed (ds_*) operations (rocprofv3's LdsUtil: the busy
    cycles summed over the CUs over elapsed cycles x CUs), bytes read and written by ds_*
    instructions per CU and elapsed cycle, the busy share of the vector memory path's address
    (TA) and data (TD) units, and the share of cycles with their queues full."""
    csv_path = os.path.join(d, "lds_counter_collection.csv")
    if not os.path.exists(csv_path):
        return []
    cus = SIMDS // 4
    rows = []
    for k, ds in _counters_by_dispatch(csv_path).items():
        ds = [e for e in ds if e["dur_ns"] >= 20000]
        if not ds or k.startswith("__amd"):
            continue
        mean = lambda key: float(np.mean([e.get(key, 0.0) for e in ds]))
        dur, elapsed = mean("dur_ns"), mean("GRBM_GUI_ACTIVE") / XCDS  # cycles at the seen clock
        if elapsed <= 0:
            continue
        per_cu = lambda key: mean(key) / (cus * elapsed)
        act = mean("SQ_LDS_IDX_ACTIVE")
        rows.append((dur, f"| `{k}` | {dur / 1e3:.1f} | {elapsed / dur:.2f} | {100 * per_cu('SQ_LDS_IDX_ACTIVE'):.1f}% | "
                          f"{64 * per_cu('SQ_INSTS_LDS_LOAD_BANDWIDTH'):.1f} | "
                          f"{64 * per_cu('SQ_INSTS_LDS_STORE_BANDWIDTH'):.1f} | "
                          f"{100 * mean('SQ_LDS_BANK_CONFLICT') / act if act > 0 else 0.0:.1f}% | "
                          f"{100 * per_cu('SQ_LDS_DATA_FIFO_FULL'):.1f}% | "
                          f"{100 * mean('TA_BUSY_avr') / elapsed:.1f}% | {100 * per_cu('TD_TD_BUSY_sum'):.1f}% | "
                          f"{100 * per_cu('SQ_VMEM_TA_ADDR_FIFO_FULL'):.1f}% |"))
    if not rows:
        return []
    return ["", "## LDS and vector-memory occupancy", "", "```", PROFILE_COMMANDS["lds"], "```", "",
            "Per kernel, the mean over its dispatches of at least 20 us; shares are of the cycles that "
            "elapsed at the seen clock (GRBM_GUI_ACTIVE / 8), per CU.  LDS busy: SQ_LDS_IDX_ACTIVE (cycles the "
            "LDS serves ds_* operations; rocprofv3's LdsUtil); LDS read/written: 64 x "
            "SQ_INSTS_LDS_LOAD/STORE_BANDWIDTH bytes per CU per cycle (ds_* instructions only: the copies "
            "from global memory straight into LDS are not among them); TA and TD busy: TA_BUSY_avr (mean over "
            "the TA instances) and TD_TD_BUSY_sum over the CUs; queue full: SQ_LDS_DATA_FIFO_FULL and "
            "SQ_VMEM_TA_ADDR_FIFO_FULL over the CUs.", "",
            "| kernel | us | clock GHz | LDS busy | LDS read B/clk | LDS written B/clk | LDS conflict | "
            "LDS data queue full | TA busy | TD busy | TA address queue full |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"] + [r for _, r in sorted(rows, key=lambda x: -x[0])]


def _summarize_gqa(d: str) -> list:
    """The float16 attention kernel of the headline (one query head per K/V head) beside the
    grouped-query workload's (five query heads per K/V head): fetched bytes per launch against
    the packed K/V bytes they cover, and the L2 hit rate, from the fetch/l2 and gqa_fetch/gqa_l2
    runs (each run's FETCH_SIZE scaled by its own closing copy)."""
    runs = [("video, 40 query heads on 40 K/V heads", "fetch", "l2", 40, 1),
            ("grouped-query, 2 x 40 query heads on 2 x 8 K/V heads", "gqa_fetch", "gqa_l2", 16, 5)]  # kv heads, group
    copy = "__amd_rocclr_copyBuffer"
    rows = []
    for title, fname, lname, kv_heads, group in runs:
        fcsv = os.path.join(d, f"{fname}_counter_collection.csv")
        lcsv = os.path.join(d, f"{lname}_counter_collection.csv")
        if not (os.path.exists(fcsv) and os.path.exists(lcsv)):
            return []
        fe, l2 = _counters_by_dispatch(fcsv), _counters_by_dispatch(lcsv)
        scale = COPY_BYTES / (sum(e.get("FETCH_SIZE", 0.0) for e in fe.get(copy, [])) * 1024.0)
        name = next((k for k in fe if k.startswith(ATTN_KERNEL) and k.endswith("true, false>")), None)
        if name is None:
            return []
        fd = [e for e in fe[name] if e["dur_ns"] >= 20000]
        ld = [e for e in l2.get(name, []) if e["dur_ns"] >= 20000]
        fetch = float(np.mean([e["FETCH_SIZE"] for e in fd])) * 1024.0 * scale
        hit = float(np.mean([e["TCC_HIT_sum"] for e in ld]))
        miss = float(np.mean([e["TCC_MISS_sum"] for e in ld]))
        dur = float(np.mean([e["dur_ns"] for e in ld]))
        # packed K/V: the token tiles (ceil(S/64) when clusters fill their tiles) and the
        # centroid tiles (256 clusters / 64), 64 keys x 128 features x 2 bytes x 2 (K and V)
        packed = kv_heads * (math.ceil(32760 / 64) + 4) * 64 * 128 * 2 * 2
        rows.append(f"| {title} | {group} | {dur / 1e3:.0f} | {packed / 1e9:.3f} | {fetch / 1e9:.2f} | "
                    f"{fetch / (kv_heads * group) / 1e9:.3f} | {100 * hit / (hit + miss):.1f}% |")
    return ["", "## K/V tiles shared by the query heads of a group", "", "```", PROFILE_COMMANDS["gqa_fetch"],
            PROFILE_COMMANDS["gqa_l2"], "```", "",
            "The float16 attention kernel, mean over its launches; the first row from the `fetch` and `l2` runs "
            "above.  The units of a group's query heads (same mask row, same tiles) run next to each other on "
            "one XCD, so their tile copies meet in its L2.", "",
            "| workload | query heads per K/V head | us | packed K/V GB | fetched GB per launch | "
            "fetched GB per query head | L2 hit |", "|---|---:|---:|---:|---:|---:|---:|"] + rows


def summarize_profiles(d: str) -> int:
    """Write the kernel-trace table, the HBM counter table and the attention kernel's traffic
    record (profiles/) from the csv files of the PROFILE_COMMANDS runs in directory d."""
    import csv

    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    stem = "wan_S32760_H40_D128"
    _summarize_trace(os.path.join(d, "trace_partitioned_kernel_trace.csv"), "trace_partitioned",
                     os.path.join(out_dir, f"partitioned_kernels_{stem}.md"),
                     "partitioned (SparsePR) call, video workload (B=1, H=40, S=32760, D=128, bf16)")
    _summarize_counters(d, os.path.join(out_dir, f"sq_l2_counters_{stem}.md"))
    trace = os.path.join(d, "trace_kernel_trace.csv")
    if os.path.exists(trace):
        calls, warm = TRACE_STEPS + TRACE_WARMUP, TRACE_WARMUP
        per = {}  # kernel -> durations in dispatch order (us)
        with open(trace) as f:
            for r in csv.DictReader(f):
                per.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
                    (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        lines = [f"# Kernel trace: whole path, video workload (B=1, H=40, S=32760, D=128, bf16)", "",
                 "Command (from the repository root, on one MI355X):", "", "```", PROFILE_COMMANDS["trace"], "```", "",
                 f"The run makes {calls} path calls: {warm} warm-up calls, then the {TRACE_STEPS} timed calls.  Each "
                 f"kernel launched a whole number of times per call is summarized over the launches of the timed "
                 f"calls only (its first {warm}/{calls} of launches dropped); durations in microseconds.", "",
                 "| kernel | launches per call | timed launches | avg us | min us | max us |",
                 "|---|---:|---:|---:|---:|---:|"]
        per_call_total = {}
        for k, ds in sorted(per.items(), key=lambda kv: -sum(x for _, x in kv[1])):
            ds.sort()
            if len(ds) % calls:
                lines.append(f"| `{k}` | ? | {len(ds)} (all) | {np.mean([x for _, x in ds]):.1f} | "
                             f"{min(x for _, x in ds):.1f} | {max(x for _, x in ds):.1f} |")
                continue
            m = len(ds) // calls
            timed = [x for _, x in ds[warm * m:]]
            per_call_total[k] = sum(timed) / TRACE_STEPS
            lines.append(f"| `{k}` | {m} | {len(timed)} | {np.mean(timed):.1f} | {min(timed):.1f} | {max(timed):.1f} |")
        attn = sum(v for k, v in per_call_total.items() if k.startswith(ATTN_KERNEL))
        stage = sum(v for k, v in per_call_total.items() if k.startswith(ATTN_KERNEL) or k.split("<")[0] in
                    ("tile_list_wave_kernel", "tile_list_kernel", "group_rank_kernel", "order_kernel"))
        lines += ["", f"Attention kernels (`{ATTN_KERNEL}`, all variants) per timed call: {attn:.1f} us; with the "
                  f"tile-list and work-order kernels of the attention stage: {stage:.1f} us."]
        # The bench line the same run printed: its attention time from HIP events on the
        # kernel's stream, against the trace's average above.
        line_path = os.path.join(d, "trace_bench.json")
        if os.path.exists(line_path):
            with open(line_path) as f:
                rows = [json.loads(x) for x in f if x.startswith("{")]
            if rows:
                rl = rows[-1]["roofline"]
                lines += ["", f"The bench line of the same run (HIP events around the timed calls): attention "
                          f"{rl['avg_launch_ms'] * 1e3:.1f} us per launch, {rl['achieved']:.1f} TFLOP/s, "
                          f"frac {rl['frac']:.4f}."]
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


def _cluster_sizes(res, cfg):
    """Query and key cluster sizes of every mask row's layout, each [B, Hm, C] float64: one
    layout shared by every head, or (partitioned path) one per (batch, K/V head)."""
    import torch

    keep = res.mask.keep
    B, Hm = keep.shape[:2]
    nk = res.layout.counts.to(torch.float64)
    qlay = res.extras.get("q_layout")
    nq = (qlay.counts if qlay is not None else res.layout.counts).to(torch.float64)
    if nk.dim() == 1:
        return nq.expand(B, Hm, -1), nk.expand(B, Hm, -1)
    kvh = torch.arange(Hm, device=keep.device) // ((cfg.Hq // cfg.Hkv) if Hm == cfg.Hq else 1)
    idx = torch.arange(B, device=keep.device)[:, None] * cfg.Hkv + kvh[None, :]
    return nq[idx], nk[idx]


def executed_pairs(res, cfg):
    """Kept token pairs per call (sum over heads and query clusters of n_a times the kept key
    tokens) -- a measurement of the mask, computed with torch on the GPU."""
    import torch

    keep = res.mask.keep.to(torch.float64)  # [B, Hm, Cq, Ck]
    nq, nk = _cluster_sizes(res, cfg)  # [B, Hm, C]
    kept_keys = (keep * nk[:, :, None, :]).sum(dim=-1)  # [B, Hm, Cq]
    per_mask_head = (kept_keys * nq).sum(dim=-1)  # [B, Hm]
    Hm = keep.shape[1]
    heads_per_mask = cfg.Hq // Hm
    return float(per_mask_head.sum().item()) * heads_per_mask


def cpu_baseline(wl, seconds_hint=20.0):
    """The float64 oracle on a bounded sample: head 0, its scores and mask, and the attention
    rows of every 2nd query cluster (plus the probe rows and the fit when the workload has
    them)."""
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
                   f"({len(clusters)} of {wl.C} query clusters)"
                   + (f", {wl.probes} dense probe rows, ridge fit" if wl.probes else "") + f"; {elapsed:.1f} s"),
        "seconds": elapsed,
    }


def measure_centroids(bsa, k, v, layout, reps=20):
    """The centroid sums on their own (bsa_centroids: read K and V once through the cluster
    layout, write the float32 means), timed with events on the current stream; GB/s over the
    K and V bytes it must read, the stage's algorithmic bytes."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api

    stream = torch.cuda.current_stream()
    api.centroids(k, v, layout)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        api.centroids(k, v, layout)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = (k.numel() + v.numel()) * k.element_size()
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBS, 4)}


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
    out = torch.empty_like(q)
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
        api.block_sparse_attention(q, kv, res.layout, res.mask, cfg.compensate, cfg.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        print(f"[profile] attention {i}", flush=True)
    for i in range(reps):
        api.pooled_qk(q, k)
        torch.cuda.synchronize()
        print(f"[profile] pooled_qk {i}", flush=True)
    for i in range(reps):
        api.response_partition(q, k, cfg.C, cfg.C, cfg.scale)
        torch.cuda.synchronize()
        print(f"[profile] response partition {i}", flush=True)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=q.device).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[profile] copy {COPY_BYTES} bytes", flush=True)
    return 0


def profile_gqa(bsa, reps):
    """The grouped-query workload (B=2, 40 query heads on 8 K/V heads, masks pooled per group):
    one path call for its layout and masks, `reps` launches of its compensated attention alone,
    then one plain device copy of COPY_BYTES."""
    import torch
    from block_sparse_attention_antidiagonal_amd import api
    from synthetic import make_config

    wl4 = make_config(4)
    cfg4 = bsa.PathConfig.from_workload(dataclasses.replace(wl4, probes=0))
    path4 = bsa.SparseAttentionPath(cfg4)
    q4 = torch.from_numpy(wl4.q).to(torch.bfloat16).cuda()
    k4 = torch.from_numpy(wl4.k).to(torch.bfloat16).cuda()
    v4 = torch.from_numpy(wl4.v).to(torch.bfloat16).cuda()
    res = path4(q4, k4, v4)
    torch.cuda.synchronize()
    kv = api.kv_pack(k4, v4, res.layout)
    ws = api.attention_workspace(q4, kv, res.layout, res.mask)
    out = torch.empty_like(q4)
    for i in range(reps):
        api.block_sparse_attention(q4, kv, res.layout, res.mask, True, cfg4.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        print(f"[profile] grouped-query attention {i}", flush=True)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=q4.device).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[profile] copy {COPY_BYTES} bytes", flush=True)
    return 0


def time_path(path, q, k, v, steps, warmup):
    """Warm up, then time `steps` whole path calls between two device synchronizations; per
    stage, the mean of the events each stage records on its own stream."""
    import torch

    res = None
    for _ in range(warmup):
        res = path(q, k, v)
    torch.cuda.synchronize()
    if res is None:
        res = path(q, k, v)
        torch.cuda.synchronize()
    marks = []  # per step: list of (stage, start event, end event)

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
    calls = []  # per step: events on the caller's stream before and after the call
    t0 = time.perf_counter()
    for _ in range(steps):
        sm = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        path(q, k, v, mark=recorder(sm))
        e1.record()
        calls.append((e0, e1))
        marks.append(sm)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    stages = {}
    for sm in marks:
        for name, e0, e1 in sm:
            stages.setdefault(name, []).append(e0.elapsed_time(e1))
    stages["call_median"] = float(np.median([e0.elapsed_time(e1) for e0, e1 in calls]))
    return ms_per_step, {name: float(np.mean(x)) if name != "call_median" else x for name, x in stages.items()}, res


def centroid_columns(res, cfg):
    """Centroid columns per call: for every query row, one per skipped non-empty key cluster
    (counted over all query heads)."""
    import torch

    keep = res.mask.keep.to(torch.float64)  # [B, Hm, Cq, Ck]
    nq, nk = _cluster_sizes(res, cfg)
    nonempty = (nk > 0).to(torch.float64)[:, :, None, :]
    skipped = ((1.0 - keep) * nonempty).sum(dim=-1)  # [B, Hm, Cq]
    return float((skipped * nq).sum().item()) * (cfg.Hq // keep.shape[1])


def path_figures(res, cfg, ms_per_step, stages_ms, probes):
    """Throughput and density figures of one timed path workload."""
    pairs = executed_pairs(res, cfg)
    cols = centroid_columns(res, cfg) if cfg.compensate else 0.0
    full = cfg.B * cfg.Hq * float(cfg.S) ** 2
    probe_pairs = float(cfg.B * cfg.Hq * probes * cfg.S)
    attn_ms = stages_ms["attention"]
    D = cfg.D
    return {
        "ms_per_call": round(ms_per_step, 4),
        "ms_per_call_median": round(stages_ms.get("call_median", ms_per_step), 4),  # events around each call
        "density": round(pairs / full, 4),  # kept token pairs / S^2, averaged over heads
        "density_with_probes": round((pairs + probe_pairs) / full, 4),  # + M*S per head
        "executed_pairs": pairs + probe_pairs,
        "executed_pair_TFLOPs": round(4 * D * (pairs + probe_pairs) / (ms_per_step * 1e-3) / 1e12, 2),
        "attention_ms": round(attn_ms, 4),
        "attention_TFLOPs": round(4 * D * pairs / (attn_ms * 1e-3) / 1e12, 2),
        "attention_mfma_frac": round(4 * D * pairs / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        # the same kernel counting the centroid columns too (4*D flops each)
        "attention_TFLOPs_with_centroids": round(4 * D * (pairs + cols) / (attn_ms * 1e-3) / 1e12, 2),
        "centroid_columns": cols,
        "stages_ms": {kk: round(vv, 4) for kk, vv in stages_ms.items()},
    }


def measure_repair_workloads(bsa, steps, warmup, wl2, q, k, v):
    """The hard-drop + probe-repair workload on the headline inputs, then the grouped-query
    workload (compensation + repair), each timed like the headline."""
    import torch
    from synthetic import make_config

    out = {}
    # The hard-drop repair workload is the headline's inputs with another path (the fields of
    # make_config(3) are those of make_config(2)).
    cfg3 = bsa.PathConfig.from_workload(dataclasses.replace(wl2, compensate=False, probes=64, lam=0.1, rank=16))
    path3 = bsa.SparseAttentionPath(cfg3)
    ms, st, res = time_path(path3, q, k, v, steps, warmup)
    out["video_harddrop_probe_repair"] = dict(
        workload="same inputs, hard-drop block-sparse attention + 64 probe rows + ridge fit (lambda 0.1, rank 16) "
                 "+ correction of every row", **path_figures(res, cfg3, ms, st, cfg3.probes))
    del path3, res
    print("[bench] grouped-query workload", file=sys.stderr, flush=True)
    wl4 = make_config(4)
    q4 = torch.from_numpy(wl4.q).to(torch.bfloat16).cuda()
    k4 = torch.from_numpy(wl4.k).to(torch.bfloat16).cuda()
    v4 = torch.from_numpy(wl4.v).to(torch.bfloat16).cuda()
    cfg4 = bsa.PathConfig.from_workload(wl4)
    path4 = bsa.SparseAttentionPath(cfg4)
    ms, st, res = time_path(path4, q4, k4, v4, steps, warmup)
    out["video_gqa_compensated_probe_repair"] = dict(
        workload="B=2, 40 query heads on 8 K/V heads, S=32760, D=128, bf16, Student-t values; masks pooled per K/V "
                 "group; compensated attention + 64 probe rows + ridge fit + correction",
        **path_figures(res, cfg4, ms, st, cfg4.probes))
    del path4, res, q4, k4, v4
    torch.cuda.synchronize()
    return out


def measure_partitioned(bsa, steps, warmup, wl2, q, k, v):
    """SparsePR's call on the headline inputs: response-coupled partitions per (batch, K/V
    head) into 256 key and 256 query groups, error-aware routes at 22% executed-pair density
    with the 64 probe rows' share reserved first, hard drop renormalized over the kept groups,
    the probe rows, the fit and the corrected attention -- every stage inside the timed call."""
    cfgp = bsa.PathConfig.from_workload(dataclasses.replace(wl2, compensate=False, probes=64, lam=0.1, rank=16))
    cfgp.mask_mode, cfgp.route_density = "partitioned", 0.22
    pathp = bsa.SparseAttentionPath(cfgp)
    ms, st, res = time_path(pathp, q, k, v, steps, warmup)
    fig = path_figures(res, cfgp, ms, st, cfgp.probes)
    fig["partition_ms"] = round(st["partition"], 4)
    return dict(workload="same inputs; response-coupled partitions (rK 48, rQ 64, 4 Lloyd iterations per grouping) "
                         "into 256 key and 256 query groups per (batch, K/V head); error-aware routes at 22% "
                         "executed-pair density including 64 probe rows; hard drop; ridge fit (lambda 0.1, rank 16); "
                         "correction in the attention epilogue", **fig)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path-only", action="store_true",
                    help="time the headline path only (no repair workloads or side measurements)")
    ap.add_argument("--partitioned-only", action="store_true",
                    help="time the partitioned (SparsePR) call alone and print its figures")
    ap.add_argument("--overlap", action="store_true",
                    help="run the K/V packing on a second stream beside the scores (default: before them)")
    ap.add_argument("--profile-kernels", type=int, default=0, metavar="K",
                    help="launch each kernel K times on its own, then one plain copy (for rocprofv3)")
    ap.add_argument("--profile-gqa", type=int, default=0, metavar="K",
                    help="launch the grouped-query workload's attention K times, then one plain copy (for rocprofv3)")
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

    if args.profile_gqa:
        return profile_gqa(bsa, args.profile_gqa)
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    wl = make_config(2)
    cfg = bsa.PathConfig.from_workload(wl)
    cfg.overlap = args.overlap
    path = bsa.SparseAttentionPath(cfg)
    q = torch.from_numpy(wl.q).to(torch.bfloat16).cuda()
    k = torch.from_numpy(wl.k).to(torch.bfloat16).cuda()
    v = torch.from_numpy(wl.v).to(torch.bfloat16).cuda()
    torch.cuda.synchronize()

    if args.profile_kernels:
        return profile_kernels(bsa, path, cfg, q, k, v, args.profile_kernels)
    if args.partitioned_only:
        print(json.dumps(measure_partitioned(bsa, args.steps, args.warmup, wl, q, k, v)), flush=True)
        return 0

    print("[bench] timing", file=sys.stderr, flush=True)
    ms_per_step, stages_ms, res = time_path(path, q, k, v, args.steps, args.warmup)
    fig = path_figures(res, cfg, ms_per_step, stages_ms, 0)
    pairs = executed_pairs(res, cfg)
    attn_ms = stages_ms["attention"]

    D, S, H = cfg.D, cfg.S, cfg.Hq
    value = 4 * D * pairs / (ms_per_step * 1e-3) / 1e12
    attn_flops = 4 * D * pairs
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    kv_bytes = 2 * cfg.B * cfg.Hkv * S * D * 2
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
            "tau": "per head from {0.85, 0.90, 0.95}", "density": fig["density"], "compensation": True,
        },
        "ms_per_call": round(ms_per_step, 4),
        "ms_per_call_median": fig["ms_per_call_median"],
        "density_with_probes": fig["density_with_probes"],
        "executed_pairs": pairs,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": ATTN_KERNEL + " (compensated)",
            "algorithmic_tflop_per_launch": attn_flops / 1e12,
            "avg_launch_ms": round(attn_ms, 4),
        },
        "attention_TFLOPs_with_centroids": fig["attention_TFLOPs_with_centroids"],
        "stages_ms": fig["stages_ms"],
        "stage_rates": {
            # the pack reads K and V once and writes them once as tiles
            "pack_GBps": round(2 * kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9, 1),
            "pack_hbm_frac": round(2 * kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            # the centroid sums alone must read K and V once (their algorithmic bytes)
            "centroids_GBps": round(kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9, 1),
            "centroids_hbm_frac": round(kv_bytes / (stages_ms["pack"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_GBps": round(qk_bytes / (stages_ms["scores"] * 1e-3) / 1e9, 1),
            "scores_hbm_frac": round(qk_bytes / (stages_ms["scores"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_TFLOPs": round(score_flops / (stages_ms["scores"] * 1e-3) / 1e12, 2),
            "scores_mfma_frac": round(score_flops / (stages_ms["scores"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
    }
    if not args.path_only:
        # the same sums by the standalone call (no tiles written), on the same K, V and layout
        line["centroids_standalone"] = measure_centroids(bsa, k, v, res.layout)
        print("[bench] repair workloads", file=sys.stderr, flush=True)
        line["repair_workloads"] = measure_repair_workloads(bsa, args.steps, args.warmup, wl, q, k, v)
        print("[bench] mask reuse", file=sys.stderr, flush=True)
        line["mask_reuse"] = measure_reuse(bsa, cfg, q, k, res)
        print("[bench] sliding-tile mask", file=sys.stderr, flush=True)
        line["sliding_tile_attention"] = measure_sliding_tile(bsa, cfg, wl, q, k, v)
        print("[bench] error-aware routing", file=sys.stderr, flush=True)
        line["error_aware_routing"] = measure_routing(bsa, cfg, q, k, v, res, line["config"]["density"])
        print("[bench] partitioned call", file=sys.stderr, flush=True)
        line["partitioned_sparsepr"] = measure_partitioned(bsa, args.steps, args.warmup, wl, q, k, v)
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
