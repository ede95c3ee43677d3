"""Benchmark: Top-20 over 1e8 int32 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--path topk|stats|kv|batched|batched_short|hist|
                            topk_large]

One step is one full library call (both stages; a single kernel launch)
over a resident synthetic input (seeded SplitMix64).  The default path,
`topk`, is the headline: topk_i32 with k = 20 over 1e8 int32 uniform over
the full range (seed 3).  `--path stats` measures reduce_stats_i32 (count,
sum, max, min and sum of squares in one pass) over 2^26 int32 uniform in
[-1000, 1000] (seed 2), the array whose sum, max and min are otherwise
asked for in three separate calls.  `--path kv` measures topk_kv_i32, the
key-value variant (the 20 largest values with their int64 positions, ties
by position), on the same 1e8 array as `topk`.  `--path batched` and
`--path batched_short` measure topk_batched_i32, the top-20 of every row of
the same array viewed as 1000 rows of 100,000 (streaming kernel, one
workgroup per row) or as 97,656 rows of 1,024 (one wave per row); the same
run also times topk_merge_i32 merging the rows' lists into the top-20 of
the whole, reported in `config.merge`.  `--path hist` measures
histogram_i32: 256 bins of width 2^24 over the same 1e8 array (its top
byte, the digit histogram of a radix pass).  `--path topk_large` measures
topk_i32 with k = 1000 on that array, which takes the radix-selection path
(several launches per call; the event time covers the whole call).

The input sits in HBM before timing starts.  W untimed calls, then K timed
back-to-back calls bracketed by device synchronisation and by a pair of HIP
events on the stream they are launched on; each call is one kernel launch,
so the event time over K is the kernel's average launch duration for the
roofline.  The result is checked against the CPU oracle before timing, and
the oracle itself is timed on the host cores as a reported baseline.

Prints ONE JSON line.  `value` is elements per second (higher is better);
`roofline` relates the kernel's algorithmic bytes (4 bytes per input
element plus the output) per launch to its measured duration and the 8 TB/s
HBM peak; `traffic` is the HBM byte count per launch measured with rocprofv3
counters (profiles/<path>_counters_*.json), reported only while the kernel
sources (their code; comments and blank lines aside) still match the ones
the counters were taken on.

Modes for profiling runs (no JSON line): --mode counters runs a few calls
plus a plain device copy of known size, to calibrate FETCH_SIZE/WRITE_SIZE.
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

PATHS = {
    "topk": {
        "metric": ("Top-20 over 1e8 int32: ms, elements/s, HBM GB/s as % of "
                   "8 TB/s peak"),
        "workload": "full_1e8",
        "describe": ("top-20 of 1e8 int32, uniform over the full int32 range "
                     "(SplitMix64 seed 3), resident in HBM"),
        "short": "top-20 of 1e8 int32, uniform full range, seed 3",
        "kernel": "topk_kernel",
        "sources": ["wave.hpp", "topk_kernel.hpp", "libtopk.hip"],
        "counters": "topk_counters_full_1e8_k20.json",
        "summary": "topk_full_1e8_k20.md",
        "out_bytes": 4 * K,
        "oracle_what": "top-20 by copy + std::sort",
    },
    "stats": {
        "metric": ("One-pass statistics (count, sum, max, min, sum of "
                   "squares) over 2^26 int32: elements/s, HBM GB/s as % of "
                   "8 TB/s peak"),
        "workload": "pm1000_2p26",
        "describe": ("count, sum, max, min and exact sum of squares of 2^26 "
                     "int32 uniform in [-1000, 1000] (SplitMix64 seed 2), "
                     "resident in HBM"),
        "short": "statistics of 2^26 int32 in [-1000, 1000], seed 2",
        "kernel": "stats_kernel",
        "sources": ["wave.hpp", "stats_kernel.hpp", "libtopk.hip"],
        "counters": "stats_counters_pm1000_2p26.json",
        "summary": "stats_pm1000_2p26.md",
        "out_bytes": 48,
        "oracle_what": "the five statistics by one loop (128-bit squares)",
    },
    "kv": {
        "metric": ("Key-value Top-20 (values + int64 positions) over 1e8 "
                   "int32: elements/s, HBM GB/s as % of 8 TB/s peak"),
        "workload": "full_1e8",
        "describe": ("top-20 of 1e8 int32 with their positions (ties by "
                     "position), uniform over the full int32 range "
                     "(SplitMix64 seed 3), resident in HBM"),
        "short": "key-value top-20 of 1e8 int32, uniform full range, seed 3",
        "kernel": "topk_kv_kernel",
        "sources": ["wave.hpp", "topk_kernel.hpp", "topk_kv_kernel.hpp",
                    "libtopk.hip"],
        "counters": "topk_kv_counters_full_1e8_k20.json",
        "summary": "topk_kv_full_1e8_k20.md",
        "out_bytes": 12 * K,
        "oracle_what": "top-20 keys by a stable sort of positions",
    },
    "batched": {
        "metric": ("Per-row Top-20 over 1e8 int32 as 1000 rows x 100,000: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "workload": "full_1e8",
        "rows": 1000, "cols": 100_000,
        "describe": ("top-20 of each of 1000 rows of 100,000 int32 (the 1e8 "
                     "array, uniform over the full int32 range, SplitMix64 "
                     "seed 3, viewed row-major), resident in HBM"),
        "short": "per-row top-20 of 1000 x 100,000 int32, seed 3",
        "kernel": "topk_kernel",
        "sources": ["wave.hpp", "topk_kernel.hpp", "libtopk.hip"],
        "counters": "topk_batched_counters_1000x100000_k20.json",
        "summary": "topk_batched_1000x100000_k20.md",
        "out_bytes": 4 * K * 1000,
        "oracle_what": "per-row top-20 by copy + std::sort of each row",
    },
    "hist": {
        "metric": ("Histogram (256 bins of width 2^24) over 1e8 int32: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "workload": "full_1e8",
        "describe": ("256-bin histogram (bins of width 2^24 from INT32_MIN: "
                     "the top byte) of 1e8 int32 uniform over the full int32 "
                     "range (SplitMix64 seed 3), resident in HBM"),
        "short": "256-bin histogram of 1e8 int32, uniform full range, seed 3",
        "kernel": "hist_kernel",
        "sources": ["wave.hpp", "hist_kernel.hpp", "libtopk.hip"],
        "counters": "hist_counters_full_1e8_256.json",
        "summary": "hist_full_1e8_256.md",
        "out_bytes": 8 * 256,
        "oracle_what": "the 256 counts by one loop",
    },
    "topk_large": {
        "metric": ("Top-1000 over 1e8 int32 (radix selection): elements/s, "
                   "HBM GB/s as % of 8 TB/s peak"),
        "workload": "full_1e8",
        "describe": ("top-1000 of 1e8 int32, uniform over the full int32 "
                     "range (SplitMix64 seed 3), resident in HBM"),
        "short": "top-1000 of 1e8 int32, uniform full range, seed 3",
        "kernel": "filter_kernel",
        "sources": ["wave.hpp", "hist_kernel.hpp", "select_kernel.hpp",
                    "libtopk.hip"],
        "counters": "topk_large_counters_full_1e8_k1000.json",
        "summary": "topk_large_full_1e8_k1000.md",
        "out_bytes": 4 * 1000,
        "oracle_what": "top-1000 by copy + std::sort",
        "k": 1000,
        # One call is eight launches: the sample, the filter pass, four
        # selection passes and the gather (these return at once after a
        # small filter copy) and the finish kernel (once per call);
        # summaries are per call.
        "call_kernels": ["sample_kernel", "filter_kernel",
                         "select_pass_kernel", "gather_kernel",
                         "select_finish_kernel"],
        "once_per_call": "select_finish_kernel",
    },
    "batched_short": {
        "metric": ("Per-row Top-20 over 1e8 int32 as 97,656 rows x 1,024: "
                   "elements/s, HBM GB/s as % of 8 TB/s peak"),
        "workload": "full_1e8",
        "rows": 97_656, "cols": 1024,
        "describe": ("top-20 of each of 97,656 rows of 1,024 int32 (the "
                     "first 99,999,744 elements of the 1e8 array, uniform "
                     "over the full int32 range, SplitMix64 seed 3, viewed "
                     "row-major), resident in HBM"),
        "short": "per-row top-20 of 97,656 x 1,024 int32, seed 3",
        "kernel": "topk_rows_kernel",
        "sources": ["wave.hpp", "topk_rows_kernel.hpp", "libtopk.hip"],
        "counters": "topk_rows_counters_97656x1024_k20.json",
        "summary": "topk_rows_97656x1024_k20.md",
        "out_bytes": 4 * K * 97_656,
        "oracle_what": "per-row top-20 by copy + std::sort of each row",
    },
}


def workload_size(P) -> int:
    import synth
    if "rows" in P:
        return P["rows"] * P["cols"]
    return synth.WORKLOADS[P["workload"]]["n"]


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
    """HBM bytes per launch from committed counter runs, if still valid."""
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
    return (
        "rocprofv3 --kernel-trace --stats -d <run>/trace -o trace "
        "--output-format csv -- python3 bench.py --steps 200 --warmup 20 "
        "--no-cpu-baseline" + flag,
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
    bytes.
    """
    import csv
    import glob

    import synth

    P = PATHS[path]
    kern = P["kernel"]

    def rows(pattern):
        files = glob.glob(os.path.join(run_dir, pattern), recursive=True)
        if not files:
            raise SystemExit("missing %s under %s" % (pattern, run_dir))
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    n = workload_size(P)
    copy_bytes = 4 * n
    algo = 4 * n + P["out_bytes"]

    call_kernels = P.get("call_kernels")

    def counter(pattern, name):
        per = {}
        for r in rows(pattern):
            if r["Counter_Name"] != name:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        mine = [v for kname, v in per.items() if kern in kname]
        copy = [v for kname, v in per.items() if "copyBuffer" in kname]
        if not mine or not copy:
            raise SystemExit("counter %s: kernels not found" % name)
        if call_kernels:
            # Per call: every dispatch of the call's kernels, divided by
            # the number of calls.
            calls = sum(len(v) for kname, v in per.items()
                        if P["once_per_call"] in kname)
            total = sum(sum(v) for kname, v in per.items()
                        if any(c in kname for c in call_kernels))
            return (total / calls, sum(copy[0]) / len(copy[0]),
                    "one call (%s)" % ", ".join(call_kernels))
        return (sum(mine[0]) / len(mine[0]), sum(copy[0]) / len(copy[0]),
                [kname for kname in per if kern in kname][0])

    fetch_k, fetch_copy, kname = counter("fetch/**/*counter_collection.csv",
                                         "FETCH_SIZE")
    write_k, write_copy, _ = counter("write/**/*counter_collection.csv",
                                     "WRITE_SIZE")
    f_scale = copy_bytes / fetch_copy   # bytes per counted unit (read side)
    w_scale = copy_bytes / write_copy   # bytes per counted unit (write side)
    traffic = fetch_k * f_scale + write_k * w_scale

    stats = rows("trace/**/*kernel_stats.csv")
    krow = [r for r in stats if kern in r["Name"]][0]
    cmd_trace, cmd_fetch, cmd_write = commands(path)
    os.makedirs(out_dir, exist_ok=True)
    data = {
        "kernel": kname,
        "workload": P["short"],
        "kernel_source_hash": kernel_source_hash(path),
        "fetch_size_kib_per_dispatch": fetch_k,
        "write_size_kib_per_dispatch": write_k,
        "copy_calibration": {
            "bytes_read_and_written": copy_bytes,
            "fetch_size_kib": fetch_copy, "write_size_kib": write_copy,
            "bytes_per_fetch_unit": f_scale, "bytes_per_write_unit": w_scale},
        "traffic_bytes_per_launch": round(traffic),
        "algorithmic_bytes_per_launch": algo,
        "commands": [cmd_fetch, cmd_write],
    }
    with open(os.path.join(out_dir, P["counters"]), "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    lines = [
        "# %s on %s" % (kern, P["short"]),
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
    avg_ns = float(krow["AverageNs"])
    what_avg = "%s average" % kern
    if call_kernels:
        calls = sum(int(r["Calls"]) for r in stats
                    if P["once_per_call"] in r["Name"])
        avg_ns = sum(int(r["Calls"]) * float(r["AverageNs"]) for r in stats
                     if any(c in r["Name"] for c in call_kernels)) / calls
        what_avg = "one call (%s, summed)" % ", ".join(call_kernels)
    lines += [
        "",
        "%s: %.2f us -> algorithmic %.0f GB/s (%.1f %% of "
        "8 TB/s)." % (what_avg, avg_ns / 1e3, algo / avg_ns,
                      100 * algo / avg_ns / 8000.0),
        "",
        "HBM traffic (rocprofv3 --pmc, one counter per run):",
        "",
        "    " + cmd_fetch,
        "    " + cmd_write,
        "",
        "| counter | %s (KiB/%s) | %d MB copy (KiB) | bytes per "
        "unit | %s bytes |" % (kern, "call, all kernels" if call_kernels
                               else "dispatch", copy_bytes // 10 ** 6, kern),
        "|---|---|---|---|---|",
        "| FETCH_SIZE | %.1f | %.1f | %.4f | %.0f |" % (
            fetch_k, fetch_copy, f_scale, fetch_k * f_scale),
        "| WRITE_SIZE | %.1f | %.1f | %.4f | %.0f |" % (
            write_k, write_copy, w_scale, write_k * w_scale),
        "",
        "Traffic per %s: %.0f bytes = %.4f x the algorithmic bytes "
        "(4 per input element + %d out)." % (
            "call" if call_kernels else "launch", traffic, traffic / algo,
            P["out_bytes"]),
        "",
    ]
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
    """Issue counters of the measured kernel (rocprofv3 --pmc, one pass per
    line of BUSY_PASSES over --mode counters) into a short summary."""
    import csv
    import glob

    P = PATHS[path]
    kern = P["kernel"]
    n = workload_size(P)
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
        "# Issue counters: %s on %s" % (kern, P["short"]),
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


def time_oracle(fn, budget_s=12.0, max_reps=3):
    """Median wall time of a single-threaded CPU oracle call."""
    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    return statistics.median(times), len(times)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--path", choices=sorted(PATHS), default="topk")
    ap.add_argument("--mode", choices=["bench", "counters"], default="bench")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    x = synth.workload(P["workload"])
    if "rows" in P:
        x = x[:P["rows"] * P["cols"]]
    n = x.size
    xd = torch.from_numpy(x).to(dev)
    stream = torch.cuda.current_stream(dev)
    if "rows" in P:
        x2 = x.reshape(P["rows"], P["cols"])
        xd2 = xd.view(P["rows"], P["cols"])
        out = torch.empty((P["rows"], K), dtype=torch.int32, device=dev)

        def call():
            return ltk.topk_batched(xd2, K, out=out)
    elif args.path == "topk":
        out = torch.empty(K, dtype=torch.int32, device=dev)

        def call():
            return ltk.topk(xd, K, out=out)
    elif args.path == "kv":
        outs = (torch.empty(K, dtype=torch.int32, device=dev),
                torch.empty(K, dtype=torch.int64, device=dev))

        def call():
            return ltk.topk_kv(xd, K, out=outs)
    elif args.path == "hist":
        out = torch.empty(256, dtype=torch.int64, device=dev)

        def call():
            return ltk.histogram(xd, -2 ** 31, 24, 256, out=out)
    elif args.path == "topk_large":
        out = torch.empty(P["k"], dtype=torch.int32, device=dev)

        def call():
            return ltk.topk(xd, P["k"], out=out)
    else:
        out = torch.empty(6, dtype=torch.int64, device=dev)

        def call():
            return ltk.stats(xd, out=out)

    if args.mode == "counters":
        # A plain copy of known size (calibrates the counters), then a few
        # launches of the measured kernel.
        src = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        print("counters mode: copy %d bytes read + %d written; 5 %s calls "
              "over n=%d" % (4 * n, 4 * n, args.path, n), flush=True)
        return

    # Correctness first (the oracle is the CPU reference; test-only code).
    import oracle
    if "rows" in P:
        got = call().cpu().numpy()
        t_rows = time.perf_counter()
        want = oracle.topk_batched(x2, K)
        t_rows = time.perf_counter() - t_rows   # the baseline: one call
        ok = np.array_equal(got, want)
    elif args.path in ("topk", "topk_large"):
        kk = P.get("k", K)
        got = call().cpu().numpy()
        want = oracle.topk(x, kk)
        ok = np.array_equal(got, want)
    elif args.path == "hist":
        got = call().cpu().numpy()
        want = oracle.histogram(x, -2 ** 31, 24, 256)
        ok = np.array_equal(got, want)
    elif args.path == "kv":
        gv, gi = call()
        got = (gv.cpu().numpy(), gi.cpu().numpy())
        t_kv = time.perf_counter()
        want = oracle.topk_kv(x, K)
        t_kv = time.perf_counter() - t_kv   # the baseline: one oracle call
        ok = (np.array_equal(got[0], want[0])
              and np.array_equal(got[1], want[1]))
    else:
        got = ltk.unpack_stats(call())
        want = oracle.stats(x)
        ok = got == want
    if not ok:
        print("MISMATCH against the oracle", got, want, file=sys.stderr)
        sys.exit(3)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # Timed region: K back-to-back calls on the stream, bracketed by device
    # synchronisation (wall clock) and by a pair of HIP events recorded on
    # the same stream.  Each call is exactly one kernel launch, so the event
    # time divided by K is the kernel's average launch duration (including
    # the short gaps between back-to-back launches).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = n * args.steps / wall

    algo_bytes = 4 * n + P["out_bytes"]
    achieved = algo_bytes / (avg_launch_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4),
        "traffic": measured_traffic(args.path),
    }

    merge = None
    if "rows" in P:
        # The rows' top-20 lists merged into the top-20 of the whole array,
        # checked against the oracle's merge of its own row results, then
        # timed the same way (one launch per call).
        mout = torch.empty(K, dtype=torch.int32, device=dev)
        got_m = ltk.topk_merge(out, K, out=mout).cpu().numpy()
        if not np.array_equal(got_m, oracle.topk_merge(want, K)):
            print("MISMATCH in the merge", got_m, file=sys.stderr)
            sys.exit(3)
        for _ in range(args.warmup):
            ltk.topk_merge(out, K, out=mout)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            ltk.topk_merge(out, K, out=mout)
        ev1.record(stream)
        torch.cuda.synchronize()
        merge = {"lists": P["rows"], "len": K, "k": K,
                 "kernel_ms_avg": round(ev0.elapsed_time(ev1) / args.steps,
                                        5)}

    cpu = None
    if not args.no_cpu_baseline:
        if "rows" in P:
            t_med, reps = t_rows, 1
            what = "the full workload (%d x %d int32, seed 3)" % (
                P["rows"], P["cols"])
        elif args.path in ("topk", "topk_large"):
            kk = P.get("k", K)
            t_med, reps = time_oracle(lambda: oracle.topk(x, kk))
            what = "the full workload (1e8 int32, seed 3)"
        elif args.path == "hist":
            t_med, reps = time_oracle(
                lambda: oracle.histogram(x, -2 ** 31, 24, 256), budget_s=10.0,
                max_reps=50)
            what = "the full workload (1e8 int32, seed 3)"
        elif args.path == "kv":
            t_med, reps = t_kv, 1
            what = "the full workload (1e8 int32, seed 3)"
        else:
            # one pass takes ~0.05 s: repeat it for about 10 s of CPU work
            t_med, reps = time_oracle(lambda: oracle.stats(x), budget_s=10.0,
                                      max_reps=250)
            what = "the full workload (2^26 int32, seed 2)"
        cpu = {
            "value": round(n / t_med, 1),
            "unit": "elements/s",
            "cores": 1,
            "kind": "oracle",
            "sample": "%s, %s on one thread; median of %d run(s) of %.2f s; "
                      "host %s, %d logical CPUs"
                      % (what, P["oracle_what"], reps, t_med, cpu_model(),
                         os.cpu_count() or 0),
        }

    config = {"workload": P["describe"], "n": n}
    if "rows" in P:
        config.update({"rows": P["rows"], "cols": P["cols"], "k": K,
                       "merge": merge})
    if args.path in ("topk", "kv"):
        config["k"] = K
    if args.path == "topk_large":
        config["k"] = P["k"]
        config["launches_per_call"] = 8
    if args.path == "hist":
        config.update({"lo": -2 ** 31, "shift": 24, "nbins": 256})
    if "rows" not in P:
        config["grid"] = ltk.grid_for(n)
    config.update({
        "kernel_ms_avg": round(avg_launch_ms, 5),
        "hbm_gbps_per_step": round(algo_bytes / (ms_per_step * 1e-3) / 1e9, 1),
    })
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
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
