"""Benchmark of libtopk on one MI355X: Top-20 over 1e8 int32 by default.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--path NAME]

Paths (each prints ONE JSON line):
  topk           top-20 of 1e8 int32, uniform over the full range, seed 3
                 (the headline workload; the default)
  c1             top-20, sum, max and min of 1e6 int32, full range, seed 1
  c2             sum, max and min of 2^26 int32 uniform in [-1000, 1000],
                 seed 2
  c4             top-100 of 1e7 int32 uniform in [0, 1000), seed 4: the
                 values as drawn, sorted ascending, and all equal
  c5             top-20 and sum of 1e9 int32, full range, seed 5 (4 GB
                 resident in HBM)
  stats          count, sum, max, min and sum of squares of the c2 array in
                 one pass (reduce_stats_i32)
  kv             key-value top-20 (values and int64 positions) of the 1e8
                 array
  batched        per-row top-20 of the 1e8 array as 1000 rows of 100,000;
                 the rows' lists are then merged (topk_merge_i32, timed
                 separately in config.merge)
  batched_short  the same as 97,656 rows of 1,024
  hist           256-bin histogram (bins of width 2^24: the top byte) of
                 the 1e8 array
  topk_large     top-1000 of the 1e8 array (radix selection, several
                 launches per call)
  segmented      per-segment top-20 of the 1e8 array cut into segments of
                 log-uniform lengths in [16, 2^18] (numpy PCG64, seed 11)

A step is one pass of the path's library calls over its input, which sits
in HBM before anything is timed.  Results are first checked against the
CPU oracle (bit-exact; the 1e9 top-k with the oracle's linear
characterisation).

Warm timing (the timed region of the JSON line): W untimed steps, then
exactly K steps back to back, bracketed by device synchronisation.
`value` is elements per second over that wall-clock region and
`ms_per_step` its wall time per step.  HIP events recorded on the stream
the calls are launched on, around every call, give each call's average
duration; `roofline` relates the dominant kernel's algorithmic bytes (4
per input element plus the output) per launch to that average ("basis"
says so) and to the 8 TB/s HBM peak.  `traffic` is the HBM byte count per
launch from committed rocprofv3 counter runs (profiles/), reported only
while the kernel sources (code, not comments) still match the ones the
counters were taken on.

Cold timing (`cold`): after the warm region, R more steps, each call
preceded, untimed, by a read of an unrelated 1 GiB buffer (written once
beforehand) on the same stream, which evicts the input from the L2 caches
and the 256 MB MALL; events around each call give its duration; medians
and minima over the R steps are reported.  Inputs smaller than the MALL
(c1, c2, c4) are served partly from it when warm.  (A flush that also
writes the buffer leaves dirty lines whose write-back the next call pays:
top-20 of 1e8 measured 71.4 us after one against 65.1 us warm.)

`cpu_baseline` times the oracle (single-threaded C++, not tuned) on the
host doing what one step does, on a bounded sample: the whole workload
(median of 3 runs), except c5, whose sample is its first 1e8 elements (one
run).

Modes for profiling runs (no JSON line): --mode counters runs a plain
device copy of the input's size (to calibrate FETCH_SIZE/WRITE_SIZE), then
five steps; --summarize / --summarize-busy turn rocprofv3 output into the
summaries under profiles/.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
K = 20
FLUSH_BYTES = 1 << 30

TOPK_SOURCES = ["wave.hpp", "topk_kernel.hpp", "libtopk.hip"]
REDUCE_SOURCES = ["wave.hpp", "reduce_kernel.hpp", "libtopk.hip"]

# calls: (label, kind, args) per step; kind: topk | reduce | stats | kv |
# batched | hist.  groups: (kernel name substring, calls it serves); the
# first group is the dominant kernel of the roofline.  Names are qualified
# (PyTorch has reduction kernels of its own called reduce_kernel).
PATHS = {
    "topk": {
        "metric": ("Top-20 over 1e8 int32: ms, elements/s, HBM GB/s as % of "
                   "8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "describe": ("top-20 of 1e8 int32, uniform over the full int32 range "
                     "(SplitMix64 seed 3), resident in HBM"),
        "short": "top-20 of 1e8 int32, uniform full range, seed 3",
        "calls": [("topk20", "topk", 20)],
        "groups": [("ltk::topk_kernel<", ["topk20"])],
        "sources": TOPK_SOURCES,
        "counters": "topk_counters_full_1e8_k20.json",
        "summary": "topk_full_1e8_k20.md",
    },
    "c1": {
        "metric": ("Top-20, sum, max and min over 1e6 int32: elements/s, HBM "
                   "GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e6", None)],
        "describe": ("top-20, exact int64 sum, max and min (four calls) of "
                     "1e6 int32 uniform over the full int32 range "
                     "(SplitMix64 seed 1), resident in HBM"),
        "short": "top-20, sum, max, min of 1e6 int32, full range, seed 1",
        "calls": [("topk20", "topk", 20), ("sum", "reduce", 0),
                  ("max", "reduce", 1), ("min", "reduce", 2)],
        "groups": [("ltk::topk_kernel<", ["topk20"]),
                   ("ltk::reduce_kernel<", ["sum", "max", "min"])],
        "sources": TOPK_SOURCES + ["reduce_kernel.hpp"],
        "counters": "c1_counters_full_1e6.json",
        "summary": "c1_full_1e6_topk20_reduce.md",
    },
    "c2": {
        "metric": ("Sum, max and min over 2^26 int32 in [-1000, 1000]: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("pm1000_2p26", None)],
        "describe": ("exact int64 sum, max and min (three calls) of 2^26 "
                     "int32 uniform in [-1000, 1000] (SplitMix64 seed 2), "
                     "resident in HBM"),
        "short": "sum, max, min of 2^26 int32 in [-1000, 1000], seed 2",
        "calls": [("sum", "reduce", 0), ("max", "reduce", 1),
                  ("min", "reduce", 2)],
        "groups": [("ltk::reduce_kernel<", ["sum", "max", "min"])],
        "sources": REDUCE_SOURCES,
        "counters": "reduce_counters_pm1000_2p26.json",
        "summary": "reduce_pm1000_2p26.md",
    },
    "c4": {
        "metric": ("Top-100 over 1e7 int32 in [0, 1000) as drawn, sorted "
                   "and all equal: elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("dup1000_1e7", None), ("dup1000_1e7", "sorted"),
                   ("dup1000_1e7", "equal")],
        "describe": ("top-100 of 1e7 int32 uniform in [0, 1000) (SplitMix64 "
                     "seed 4), of the same values sorted ascending, and of 1e7 "
                     "copies of the first value (three calls, three arrays), "
                     "resident in HBM"),
        "short": "top-100 of 1e7 int32 in [0, 1000): drawn, sorted, equal",
        "calls": [("uniform", "topk", 100, 0), ("sorted", "topk", 100, 1),
                  ("equal", "topk", 100, 2)],
        "groups": [("ltk::topk_kernel<", ["uniform", "sorted", "equal"])],
        "sources": TOPK_SOURCES,
        "counters": "c4_counters_dup1000_1e7_k100.json",
        "summary": "c4_dup1000_1e7_k100.md",
    },
    "c5": {
        "metric": ("Top-20 and sum over 1e9 int32 (4 GB in HBM): "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e9", None)],
        "describe": ("top-20 and exact int64 sum (two calls) of 1e9 int32 "
                     "uniform over the full int32 range (SplitMix64 seed 5), "
                     "4 GB resident in HBM"),
        "short": "top-20 and sum of 1e9 int32, full range, seed 5",
        "calls": [("topk20", "topk", 20), ("sum", "reduce", 0)],
        "groups": [("ltk::topk_kernel<", ["topk20"]),
                   ("ltk::reduce_kernel<", ["sum"])],
        "sources": TOPK_SOURCES + ["reduce_kernel.hpp"],
        "counters": "c5_counters_full_1e9.json",
        "summary": "c5_full_1e9_topk20_sum.md",
        "oracle_sample": 100_000_000,
        "cold_steps": 10,
    },
    "stats": {
        "metric": ("One-pass statistics (count, sum, max, min, sum of "
                   "squares) over 2^26 int32: elements/s, HBM GB/s as % of "
                   "8 TB/s peak"),
        "inputs": [("pm1000_2p26", None)],
        "describe": ("count, sum, max, min and exact sum of squares of 2^26 "
                     "int32 uniform in [-1000, 1000] (SplitMix64 seed 2), "
                     "resident in HBM"),
        "short": "statistics of 2^26 int32 in [-1000, 1000], seed 2",
        "calls": [("stats", "stats")],
        "groups": [("ltk::stats_kernel<", ["stats"])],
        "sources": ["wave.hpp", "stats_kernel.hpp", "libtopk.hip"],
        "counters": "stats_counters_pm1000_2p26.json",
        "summary": "stats_pm1000_2p26.md",
    },
    "kv": {
        "metric": ("Key-value Top-20 (values + int64 positions) over 1e8 "
                   "int32: elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "describe": ("top-20 of 1e8 int32 with their positions (ties by "
                     "position), uniform over the full int32 range "
                     "(SplitMix64 seed 3), resident in HBM"),
        "short": "key-value top-20 of 1e8 int32, uniform full range, seed 3",
        "calls": [("kv20", "kv", 20)],
        "groups": [("ltk::topk_kv_kernel<", ["kv20"])],
        "sources": ["wave.hpp", "topk_kernel.hpp", "topk_kv_kernel.hpp",
                    "libtopk.hip"],
        "counters": "topk_kv_counters_full_1e8_k20.json",
        "summary": "topk_kv_full_1e8_k20.md",
    },
    "batched": {
        "metric": ("Per-row Top-20 over 1e8 int32 as 1000 rows x 100,000: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "rows": 1000, "cols": 100_000,
        "describe": ("top-20 of each of 1000 rows of 100,000 int32 (the 1e8 "
                     "array, uniform over the full int32 range, SplitMix64 "
                     "seed 3, viewed row-major), resident in HBM"),
        "short": "per-row top-20 of 1000 x 100,000 int32, seed 3",
        "calls": [("rows20", "batched", 20)],
        "groups": [("ltk::topk_kernel<", ["rows20"])],
        "sources": TOPK_SOURCES,
        "counters": "topk_batched_counters_1000x100000_k20.json",
        "summary": "topk_batched_1000x100000_k20.md",
    },
    "batched_short": {
        "metric": ("Per-row Top-20 over 1e8 int32 as 97,656 rows x 1,024: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "rows": 97_656, "cols": 1024,
        "describe": ("top-20 of each of 97,656 rows of 1,024 int32 (the "
                     "first 99,999,744 elements of the 1e8 array, uniform "
                     "over the full int32 range, SplitMix64 seed 3, viewed "
                     "row-major), resident in HBM"),
        "short": "per-row top-20 of 97,656 x 1,024 int32, seed 3",
        "calls": [("rows20", "batched", 20)],
        "groups": [("ltk::topk_rows_kernel<", ["rows20"])],
        "sources": ["wave.hpp", "topk_rows_kernel.hpp", "libtopk.hip"],
        "counters": "topk_rows_counters_97656x1024_k20.json",
        "summary": "topk_rows_97656x1024_k20.md",
    },
    "hist": {
        "metric": ("Histogram (256 bins of width 2^24) over 1e8 int32: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "describe": ("256-bin histogram (bins of width 2^24 from INT32_MIN: "
                     "the top byte) of 1e8 int32 uniform over the full int32 "
                     "range (SplitMix64 seed 3), resident in HBM"),
        "short": "256-bin histogram of 1e8 int32, uniform full range, seed 3",
        "calls": [("hist256", "hist", (-2 ** 31, 24, 256))],
        "groups": [("ltk::hist_kernel<", ["hist256"])],
        "sources": ["wave.hpp", "hist_kernel.hpp", "libtopk.hip"],
        "counters": "hist_counters_full_1e8_256.json",
        "summary": "hist_full_1e8_256.md",
    },
    "segmented": {
        "metric": ("Segmented Top-20 over 1e8 int32 (segment lengths "
                   "log-uniform in [16, 2^18]): elements/s, HBM GB/s as % of "
                   "8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "segments": (16, 1 << 18, 11),
        "describe": ("top-20 of every segment of 1e8 int32 uniform over the "
                     "full int32 range (SplitMix64 seed 3), cut into segments "
                     "whose lengths are log-uniform in [16, 2^18] (numpy "
                     "PCG64 seed 11; 3967 segments), resident in HBM"),
        "short": "segmented top-20 of 1e8 int32, lengths log-uniform in "
                 "[16, 2^18]",
        "calls": [("seg20", "segmented", 20)],
        # One call is two launches; summaries and traffic are per call.
        "groups": [("ltk::seg_long_kernel<", ["seg20"])],
        "call_kernels": ["ltk::seg_short_kernel<", "ltk::seg_long_kernel<"],
        "once_per_call": "ltk::seg_short_kernel<",
        "launches_per_call": 2,
        "sources": ["wave.hpp", "topk_kernel.hpp", "topk_rows_kernel.hpp",
                    "seg_kernel.hpp", "libtopk.hip"],
        "counters": "seg_counters_full_1e8_k20.json",
        "summary": "seg_full_1e8_k20.md",
    },
    "topk_large": {
        "metric": ("Top-1000 over 1e8 int32 (radix selection): elements/s, "
                   "HBM GB/s as % of 8 TB/s peak"),
        "inputs": [("full_1e8", None)],
        "describe": ("top-1000 of 1e8 int32, uniform over the full int32 "
                     "range (SplitMix64 seed 3), resident in HBM"),
        "short": "top-1000 of 1e8 int32, uniform full range, seed 3",
        "calls": [("topk1000", "topk", 1000)],
        # One call is several launches; the summaries and the traffic are
        # per call: every dispatch of these kernels, divided by the number
        # of calls (one select_finish_kernel each).
        "groups": [("ltk::filter_kernel<", ["topk1000"])],
        "call_kernels": ["ltk::sample_kernel(", "ltk::filter_kernel<",
                         "ltk::select_pass_kernel<", "ltk::gather_kernel<",
                         "ltk::select_finish_kernel("],
        "once_per_call": "ltk::select_finish_kernel(",
        "launches_per_call": 8,
        "sources": ["wave.hpp", "hist_kernel.hpp", "select_kernel.hpp",
                    "libtopk.hip"],
        "counters": "topk_large_counters_full_1e8_k1000.json",
        "summary": "topk_large_full_1e8_k1000.md",
    },
}


def short_name(kern: str) -> str:
    """ltk::topk_kernel< -> topk_kernel"""
    return kern.replace("ltk::", "").rstrip("<(")


def input_size(P) -> int:
    """Elements of one input array (a matrix path: rows x cols)."""
    import synth
    if "rows" in P:
        return P["rows"] * P["cols"]
    return synth.WORKLOADS[P["inputs"][0][0]]["n"]


def call_algo_bytes(P, call) -> int:
    """Algorithmic bytes of one call: 4 per input element plus its output."""
    n = input_size(P)
    kind = call[1]
    if kind == "topk":
        return 4 * n + 4 * call[2]
    if kind == "reduce":
        return 4 * n + 8
    if kind == "stats":
        return 4 * n + 48
    if kind == "kv":
        return 4 * n + 12 * call[2]
    if kind == "batched":
        return 4 * n + 4 * call[2] * P["rows"]
    if kind == "hist":
        return 4 * n + 8 * call[2][2]
    if kind == "segmented":
        nseg = P["nseg"]
        return 4 * n + 8 * (nseg + 1) + 4 * call[2] * nseg + 4 * nseg
    raise ValueError(kind)


def group_algo_bytes(P, group) -> int:
    """Algorithmic bytes per launch of a kernel group (its calls' mean)."""
    calls = [c for c in P["calls"] if c[0] in group[1]]
    return sum(call_algo_bytes(P, c) for c in calls) // len(calls)


def code_only(text: str) -> str:
    """Source text without // comments and blank lines: edits to comments
    leave the compiled kernels, and so the counters, as they were."""
    out = []
    for line in text.splitlines():
        i = line.find("//")
        if i >= 0:
            line = line[:i]
        line = line.rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def kernel_source_hash(path: str) -> str:
    h = hashlib.sha256()
    for name in PATHS[path]["sources"]:
        with open(os.path.join(ROOT, "top_selection_two_amd", "csrc", name),
                  encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(path: str):
    """HBM bytes per launch of the dominant kernel from committed counter
    runs, if they were taken on the current kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles",
                               PATHS[path]["counters"])) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash(path):
        return None
    return c.get("traffic_bytes_per_launch")


def commands(path: str):
    flag = "" if path == "topk" else " --path %s" % path
    steps = " --steps 20 --warmup 3" if path == "c5" else \
        " --steps 200 --warmup 20"
    return (
        "rocprofv3 --kernel-trace --stats -d <run>/trace -o trace "
        "--output-format csv -- python3 bench.py%s --no-cpu-baseline"
        % steps + flag,
        "rocprofv3 --pmc FETCH_SIZE -d <run>/fetch -o fetch --output-format "
        "csv -- python3 bench.py --mode counters" + flag,
        "rocprofv3 --pmc WRITE_SIZE -d <run>/write -o write --output-format "
        "csv -- python3 bench.py --mode counters" + flag,
    )


def summarize(run_dir: str, out_dir: str, path: str) -> None:
    """Turn rocprofv3 CSV output into the committed summaries.

    run_dir holds the three profiler runs made by the commands printed in
    the summaries: trace/ (--kernel-trace --stats over a timed bench run),
    fetch/ and write/ (--pmc FETCH_SIZE, --pmc WRITE_SIZE over --mode
    counters).  The counter values (KiB per dispatch) are scaled by what the
    same counter reads for the plain device copy of the input's size that
    --mode counters runs first (torch's copy kernel), so that traffic is in
    bytes.  One row per kernel group of the path.
    """
    import csv
    import glob

    P = PATHS[path]

    def rows(pattern):
        files = glob.glob(os.path.join(run_dir, pattern), recursive=True)
        if not files:
            raise SystemExit("missing %s under %s" % (pattern, run_dir))
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    n = input_size(P)
    copy_bytes = 4 * n
    call_kernels = P.get("call_kernels")

    def per_kernel(pattern, name):
        per = {}
        for r in rows(pattern):
            if r["Counter_Name"] == name:
                per.setdefault(r["Kernel_Name"], []).append(
                    float(r["Counter_Value"]))
        copy = [v for kname, v in per.items() if "copyBuffer" in kname]
        if not copy:
            raise SystemExit("counter %s: the copy kernel is missing" % name)
        return per, sum(copy[0]) / len(copy[0])

    fetch, fetch_copy = per_kernel("fetch/**/*counter_collection.csv",
                                   "FETCH_SIZE")
    write, write_copy = per_kernel("write/**/*counter_collection.csv",
                                   "WRITE_SIZE")
    f_scale = copy_bytes / fetch_copy   # bytes per counted unit (read side)
    w_scale = copy_bytes / write_copy   # bytes per counted unit (write side)
    stats = rows("trace/**/*kernel_stats.csv")

    def group_counter(per, kern):
        if call_kernels:
            calls = sum(len(v) for kname, v in per.items()
                        if P["once_per_call"] in kname)
            return sum(sum(v) for kname, v in per.items()
                       if any(c in kname for c in call_kernels)) / calls
        vals = [x for kname, v in per.items() if kern in kname for x in v]
        if not vals:
            raise SystemExit("no %s dispatches in the counter runs" % kern)
        return sum(vals) / len(vals)

    def group_time(kern):
        if call_kernels:
            calls = sum(int(r["Calls"]) for r in stats
                        if P["once_per_call"] in r["Name"])
            return sum(int(r["Calls"]) * float(r["AverageNs"]) for r in stats
                       if any(c in r["Name"] for c in call_kernels)) / calls
        mine = [r for r in stats if kern in r["Name"]]
        calls = sum(int(r["Calls"]) for r in mine)
        return sum(int(r["Calls"]) * float(r["AverageNs"])
                   for r in mine) / calls

    groups = []
    for kern, labels in P["groups"]:
        algo = group_algo_bytes(P, (kern, labels))
        fk = group_counter(fetch, kern)
        wk = group_counter(write, kern)
        groups.append({
            "kernel": short_name(kern), "calls": labels,
            "algorithmic_bytes_per_launch": algo,
            "fetch_size_kib_per_dispatch": fk,
            "write_size_kib_per_dispatch": wk,
            "traffic_bytes_per_launch": round(fk * f_scale + wk * w_scale),
            "trace_average_ns": group_time(kern),
        })
    cmd_trace, cmd_fetch, cmd_write = commands(path)
    os.makedirs(out_dir, exist_ok=True)
    dom = groups[0]
    data = {
        "kernel": dom["kernel"],
        "workload": P["short"],
        "kernel_source_hash": kernel_source_hash(path),
        "fetch_size_kib_per_dispatch": dom["fetch_size_kib_per_dispatch"],
        "write_size_kib_per_dispatch": dom["write_size_kib_per_dispatch"],
        "copy_calibration": {
            "bytes_read_and_written": copy_bytes,
            "fetch_size_kib": fetch_copy, "write_size_kib": write_copy,
            "bytes_per_fetch_unit": f_scale, "bytes_per_write_unit": w_scale},
        "traffic_bytes_per_launch": dom["traffic_bytes_per_launch"],
        "algorithmic_bytes_per_launch": dom["algorithmic_bytes_per_launch"],
        "groups": groups,
        "commands": [cmd_fetch, cmd_write],
    }
    with open(os.path.join(out_dir, P["counters"]), "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    per = "call, all kernels" if call_kernels else "dispatch"
    lines = [
        "# %s" % P["short"],
        "",
        "Kernel trace (rocprofv3 --kernel-trace --stats), from the repository "
        "root:",
        "",
        "    " + cmd_trace,
        "",
        "| kernel | calls | average ns | min ns | max ns | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in stats:
        lines.append("| %s | %s | %s | %s | %s | %s |" % (
            r["Name"][:60], r["Calls"], r["AverageNs"], r["MinNs"],
            r["MaxNs"], r.get("Percentage", "")))
    lines += ["", "HBM traffic (rocprofv3 --pmc, one counter per run):", "",
              "    " + cmd_fetch, "    " + cmd_write, "",
              "Copy calibration: a %d MB device copy reads %.1f KiB "
              "(FETCH_SIZE) and writes %.1f KiB (WRITE_SIZE): %.4f and %.4f "
              "bytes per counted unit." % (copy_bytes // 10 ** 6, fetch_copy,
                                          write_copy, f_scale, w_scale),
              "",
              "| kernel | average us (trace) | algorithmic bytes | GB/s | "
              "%% of 8 TB/s | FETCH_SIZE KiB/%s | WRITE_SIZE KiB/%s | "
              "traffic bytes | traffic / algorithmic |" % (per, per),
              "|---|---|---|---|---|---|---|---|---|"]
    for g in groups:
        ns = g["trace_average_ns"]
        a = g["algorithmic_bytes_per_launch"]
        lines.append("| %s%s | %.2f | %d | %.0f | %.1f | %.1f | %.1f | %d | "
                     "%.4f |" % (
                         g["kernel"], " (one call, summed)" if call_kernels
                         else "", ns / 1e3, a, a / ns, 100 * a / ns / 8000.0,
                         g["fetch_size_kib_per_dispatch"],
                         g["write_size_kib_per_dispatch"],
                         g["traffic_bytes_per_launch"],
                         g["traffic_bytes_per_launch"] / a))
    lines.append("")
    with open(os.path.join(out_dir, P["summary"]), "w") as f:
        f.write("\n".join(lines))
    print("wrote summaries to", out_dir)


BUSY_PASSES = (
    ("busy", "VALUBusy SALUBusy"),
    ("insts", "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVES"),
    ("stall", "MemUnitStalled VALUUtilization"),
)


def busy_commands(path: str):
    flag = "" if path == "topk" else " --path %s" % path
    return ["rocprofv3 --pmc %s -d <run>/%s -o %s --output-format csv -- "
            "python3 bench.py --mode counters%s" % (c, d, d, flag)
            for d, c in BUSY_PASSES]


def summarize_busy(run_dir: str, out_dir: str, path: str) -> None:
    """Issue counters of the dominant kernel (rocprofv3 --pmc, one pass per
    line of BUSY_PASSES over --mode counters) into a short summary."""
    import csv
    import glob

    P = PATHS[path]
    kern = P["groups"][0][0]
    n = input_size(P)
    vals = {}
    for d, _ in BUSY_PASSES:
        files = glob.glob(os.path.join(run_dir, d, "**",
                                       "*counter_collection.csv"),
                          recursive=True)
        if not files:
            raise SystemExit("missing the %s pass under %s" % (d, run_dir))
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                if kern in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    avg = {c: sum(v) / len(v) for c, v in vals.items()}
    lines = [
        "# Issue counters: %s on %s" % (short_name(kern), P["short"]),
        "",
        "From the repository root, one rocprofv3 pass per line:",
        "",
    ] + ["    " + c for c in busy_commands(path)] + [
        "",
        "| counter | per dispatch (mean) |",
        "|---|---|",
    ]
    for c in sorted(avg):
        lines.append("| %s | %.2f |" % (c, avg[c]))
    if "SQ_INSTS_VALU" in avg:
        lines += [
            "",
            "VALU instructions per input element: %.3f (wave instructions x "
            "64 lanes / elements: %.2f lane-ops per element)."
            % (avg["SQ_INSTS_VALU"] / n, avg["SQ_INSTS_VALU"] * 64 / n),
            "SALU instructions per input element: %.3f."
            % (avg.get("SQ_INSTS_SALU", 0.0) / n),
        ]
    lines.append("")
    name = P["summary"].replace(".md", "_issue.md")
    with open(os.path.join(out_dir, name), "w") as f:
        f.write("\n".join(lines))
    print("wrote", name)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ------------------------------------------------------------------ calls
def segment_offsets(P):
    import synth
    lo, hi, seed = P["segments"]
    return synth.segment_offsets(input_size(P), lo, hi, seed)


def make_runner(ltk, P, call, xds, dev):
    """A closure that launches one library call on the current stream."""
    import torch
    kind = call[1]
    src = xds[call[3] if len(call) > 3 else 0]
    if kind == "segmented":
        offs = torch.from_numpy(segment_offsets(P)).to(dev)
        nseg = offs.numel() - 1
        out = torch.empty((nseg, call[2]), dtype=torch.int32, device=dev)
        cnt = torch.empty(nseg, dtype=torch.int32, device=dev)
        return lambda: ltk.topk_segmented(src, offs, call[2], out=out,
                                          counts=cnt)
    if kind == "topk":
        out = torch.empty(call[2], dtype=torch.int32, device=dev)
        return lambda: ltk.topk(src, call[2], out=out)
    if kind == "reduce":
        out = torch.empty(1, dtype=torch.int64, device=dev)
        return lambda: ltk.reduce(src, call[2], out=out)
    if kind == "stats":
        out = torch.empty(6, dtype=torch.int64, device=dev)
        return lambda: ltk.stats(src, out=out)
    if kind == "kv":
        outs = (torch.empty(call[2], dtype=torch.int32, device=dev),
                torch.empty(call[2], dtype=torch.int64, device=dev))
        return lambda: ltk.topk_kv(src, call[2], out=outs)
    if kind == "batched":
        m = src[:P["rows"] * P["cols"]].view(P["rows"], P["cols"])
        out = torch.empty((P["rows"], call[2]), dtype=torch.int32, device=dev)
        return lambda: ltk.topk_batched(m, call[2], out=out)
    if kind == "hist":
        lo, shift, nbins = call[2]
        out = torch.empty(nbins, dtype=torch.int64, device=dev)
        return lambda: ltk.histogram(src, lo, shift, nbins, out=out)
    raise ValueError(kind)


def oracle_result(oracle, P, call, x):
    """What the oracle computes for one call on host array x."""
    kind = call[1]
    if kind == "topk":
        return oracle.topk(x, call[2])
    if kind == "reduce":
        return oracle.reduce(x, call[2])
    if kind == "stats":
        return oracle.stats(x)
    if kind == "kv":
        return oracle.topk_kv(x, call[2])
    if kind == "batched":
        rows, cols = P["rows"], P["cols"]
        return oracle.topk_batched(x[:rows * cols].reshape(rows, cols),
                                   call[2])
    if kind == "hist":
        return oracle.histogram(x, *call[2])
    if kind == "segmented":
        return oracle.topk_segmented(x, segment_offsets(P), call[2])
    raise ValueError(kind)


def fetch_result(ltk, call, res):
    """The device result of a call, on the host, comparable with the
    oracle's."""
    import numpy as np
    kind = call[1]
    if kind == "reduce":
        return int(res.cpu()[0])
    if kind == "stats":
        return ltk.unpack_stats(res)
    if kind in ("kv", "segmented"):
        return (res[0].cpu().numpy(), res[1].cpu().numpy())
    return np.asarray(res.cpu().numpy())


def same(a, b) -> bool:
    import numpy as np
    if isinstance(a, tuple):
        return all(np.array_equal(p, q) for p, q in zip(a, b))
    if isinstance(a, (int, dict)):
        return a == b
    return np.array_equal(a, b)


# ------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--path", choices=sorted(PATHS), default="topk")
    ap.add_argument("--mode", choices=["bench", "counters"], default="bench")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold (cache-flushed) timing")
    ap.add_argument("--grid", type=int, default=0,
                    help="stage-1 workgroups (0 = library default)")
    ap.add_argument("--summarize", metavar="RUN_DIR",
                    help="write profiles/ summaries from rocprofv3 output "
                         "(CPU only)")
    ap.add_argument("--summarize-busy", metavar="RUN_DIR",
                    help="write the issue-counter summary (VALUBusy, "
                         "instructions per element) from rocprofv3 output "
                         "(CPU only)")
    args = ap.parse_args()
    P = PATHS[args.path]
    if "segments" in P:
        P["nseg"] = int(segment_offsets(P).size - 1)
    if args.summarize:
        summarize(args.summarize, os.path.join(ROOT, "profiles"), args.path)
        return
    if args.summarize_busy:
        summarize_busy(args.summarize_busy, os.path.join(ROOT, "profiles"),
                       args.path)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import top_selection_two_amd as ltk

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ltk.set_grid(args.grid)

    xs = [synth.workload(name, variant) for name, variant in P["inputs"]]
    xds = [torch.from_numpy(x).to(dev) for x in xs]
    n = input_size(P)
    stream = torch.cuda.current_stream(dev)
    calls = P["calls"]
    runners = [make_runner(ltk, P, c, xds, dev) for c in calls]

    def step():
        for r in runners:
            r()

    if args.mode == "counters":
        # A plain copy of known size (calibrates the counters), then a few
        # steps.
        src = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        print("counters mode: copy %d bytes read + %d written; 5 steps of %s "
              "over n=%d" % (4 * n, 4 * n, args.path, n), flush=True)
        return

    # ---- correctness first (the oracle is the CPU reference) ------------
    import oracle
    sample_n = P.get("oracle_sample")
    got = [fetch_result(ltk, c, r()) for c, r in zip(calls, runners)]
    torch.cuda.synchronize()
    oracle_times = []   # seconds per oracle step on the sample
    if sample_n is None:
        # The whole workload is the sample: the first timed oracle step
        # also gives the expected results.
        t0 = time.perf_counter()
        want = [oracle_result(oracle, P, c, xs[c[3] if len(c) > 3 else 0])
                for c in calls]
        oracle_times.append(time.perf_counter() - t0)
        ok = all(same(g, w) for g, w in zip(got, want))
    else:
        # Too large to sort: the linear top-k characterisation and the
        # oracle's own loops over the whole input.
        ok = True
        for c, g in zip(calls, got):
            x = xs[c[3] if len(c) > 3 else 0]
            if c[1] == "topk":
                ok &= oracle.check_topk(x, c[2], g) == 0
            else:
                ok &= same(g, oracle_result(oracle, P, c, x))
    if not ok:
        print("MISMATCH against the oracle", got, file=sys.stderr)
        sys.exit(3)

    merge = None
    if "rows" in P:
        # The rows' top-k lists merged into the top-k of the whole array,
        # checked against the oracle, then timed (one launch per call).
        mout = torch.empty(K, dtype=torch.int32, device=dev)
        rows_out = runners[0]()
        got_m = ltk.topk_merge(rows_out, K, out=mout).cpu().numpy()
        if not np.array_equal(got_m, oracle.topk_merge(got[0], K)):
            print("MISMATCH in the merge", got_m, file=sys.stderr)
            sys.exit(3)

    # ---- warm: the timed region -----------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # One call per step: a pair of events around the K calls (their
    # average includes the short gaps between back-to-back launches).
    # Several: events between the calls, to tell the kernels apart.
    nc = len(calls)
    marks = nc + 1 if nc > 1 else 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)]
           for _ in range(args.steps if nc > 1 else 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if nc == 1:
        evs[0][0].record(stream)
        for s in range(args.steps):
            runners[0]()
        evs[0][1].record(stream)
    else:
        for s in range(args.steps):
            evs[s][0].record(stream)
            for j, r in enumerate(runners):
                r()
                evs[s][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    if nc == 1:
        warm_ms = [evs[0][0].elapsed_time(evs[0][1]) / args.steps]
    else:
        warm_ms = [sum(evs[s][j].elapsed_time(evs[s][j + 1])
                       for s in range(args.steps)) / args.steps
                   for j in range(nc)]
    elements_per_step = n * nc
    value = elements_per_step * args.steps / wall

    # ---- cold: every call after a 1 GiB read + write --------------------
    cold = None
    cold_ms = None
    if not args.no_cold:
        flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        R = min(args.steps, P.get("cold_steps", 20))
        pairs = [[(torch.cuda.Event(enable_timing=True),
                   torch.cuda.Event(enable_timing=True)) for _ in range(nc)]
                 for _ in range(R)]
        torch.cuda.synchronize()
        for s in range(R):
            for j, r in enumerate(runners):
                torch.amax(flush)       # untimed: evicts L2 and MALL
                pairs[s][j][0].record(stream)
                r()
                pairs[s][j][1].record(stream)
        torch.cuda.synchronize()
        del flush
        per = [[pairs[s][j][0].elapsed_time(pairs[s][j][1]) for s in range(R)]
               for j in range(nc)]
        steps_ms = [sum(per[j][s] for j in range(nc)) for s in range(R)]
        cold_ms = [statistics.median(v) for v in per]
        med = statistics.median(steps_ms)
        cold = {
            "steps": R,
            "flush": "1 GiB read of an unrelated buffer before each call, "
                     "untimed",
            "ms_per_step_median": round(med, 5),
            "ms_per_step_min": round(min(steps_ms), 5),
            "value_median": round(elements_per_step / (med * 1e-3), 1),
            "calls_ms_median": {c[0]: round(t, 5)
                                for c, t in zip(calls, cold_ms)},
        }

    if "rows" in P:
        for _ in range(args.warmup):
            ltk.topk_merge(rows_out, K, out=mout)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            ltk.topk_merge(rows_out, K, out=mout)
        e1.record(stream)
        torch.cuda.synchronize()
        merge = {"lists": P["rows"], "len": K, "k": K,
                 "kernel_ms_avg": round(e0.elapsed_time(e1) / args.steps, 5)}

    # ---- roofline of the dominant kernel --------------------------------
    kern, labels = P["groups"][0]
    idx = [j for j, c in enumerate(calls) if c[0] in labels]
    launch_ms = sum(warm_ms[j] for j in idx) / len(idx)
    algo = group_algo_bytes(P, P["groups"][0])
    achieved = algo / (launch_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4),
        "traffic": measured_traffic(args.path),
        "kernel": short_name(kern),
        "basis": ("algorithmic bytes per launch (%d) / average %s duration "
                  "from HIP events around each call in the warm timed region"
                  % (algo, "call" if P.get("call_kernels") else "launch")),
    }
    if cold_ms is not None:
        cms = sum(cold_ms[j] for j in idx) / len(idx)
        roofline["cold_frac"] = round(algo / (cms * 1e-3) / 1e9 / PEAK_GBPS,
                                      4)

    # ---- CPU baseline: the oracle doing one step on the sample -----------
    cpu = None
    if not args.no_cpu_baseline:
        if sample_n is None:
            reps = 3
            while len(oracle_times) < reps:
                t0 = time.perf_counter()
                for c in calls:
                    oracle_result(oracle, P, c,
                                  xs[c[3] if len(c) > 3 else 0])
                oracle_times.append(time.perf_counter() - t0)
            sample_desc = "the whole workload"
            sample_elems = elements_per_step
        else:
            xsmp = xs[0][:sample_n]
            t0 = time.perf_counter()
            for c in calls:
                oracle_result(oracle, P, c, xsmp)
            oracle_times.append(time.perf_counter() - t0)
            sample_desc = ("the first %d elements of the input (one step of "
                           "the same calls on them)" % sample_n)
            sample_elems = sample_n * nc
        t_med = statistics.median(oracle_times)
        cpu = {
            "value": round(sample_elems / t_med, 1),
            "unit": "elements/s",
            "cores": 1,
            "kind": "oracle",
            "sample": "%s: %s on one thread (copy + std::sort for top-k, "
                      "int64 loops for reductions); median of %d run(s) of "
                      "%.2f s; host %s, %d logical CPUs"
                      % (sample_desc, ", ".join(c[0] for c in calls),
                         len(oracle_times), t_med, cpu_model(),
                         os.cpu_count() or 0),
        }

    config = {"workload": P["describe"], "n": n,
              "calls_per_step": [c[0] for c in calls],
              "calls_ms_avg_warm": {c[0]: round(t, 5)
                                    for c, t in zip(calls, warm_ms)}}
    if "rows" in P:
        config.update({"rows": P["rows"], "cols": P["cols"], "k": K,
                       "merge": merge})
    elif any(c[1] in ("topk", "kv") and c[2] <= ltk.max_k() for c in calls):
        # The top-k grid (the other calls size their own grids).
        config["topk_grid"] = ltk.grid_for(n)
    if P.get("launches_per_call"):
        config["launches_per_call"] = P["launches_per_call"]
    if "segments" in P:
        config["segments"] = P["nseg"]
    config["hbm_gbps_per_step"] = round(
        sum(call_algo_bytes(P, c) for c in calls) / (ms_per_step * 1e-3)
        / 1e9, 1)
    line = {
        "metric": P["metric"],
        "value": round(value, 1),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
