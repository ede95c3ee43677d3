"""Benchmark: Top-20 over 1e8 int32 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one full topk_i32 call (both stages; a single kernel launch) over
the resident 1e8-element input.  The input is synthetic (seeded SplitMix64,
uniform over the full int32 range, seed 3) and sits in HBM before timing
starts.  W untimed calls, then K timed calls bracketed by device
synchronisation; every timed call is also bracketed by its own pair of HIP
events on the stream it is launched on, which gives the kernel's average
launch duration for the roofline.  The result is checked against the CPU
oracle before timing, and the oracle itself is timed on the host cores as a
reported baseline.

Prints ONE JSON line.  `value` is elements per second (higher is better);
`roofline` relates the kernel's algorithmic bytes (4 bytes per input element
plus 4 per output element) per launch to its measured duration and the
8 TB/s HBM peak; `traffic` is the HBM byte count per launch measured with
rocprofv3 counters (profiles/topk_counters_full_1e8_k20.json), reported only
while the kernel sources still match the ones the counters were taken on.

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

METRIC = ("Top-20 over 1e8 int32: ms, elements/s, HBM GB/s as % of 8 TB/s "
          "peak")
PEAK_GBPS = 8000.0
WORKLOAD = "full_1e8"
K = 20
COUNTERS = os.path.join(ROOT, "profiles", "topk_counters_full_1e8_k20.json")
KERNEL_SOURCES = ["wave.hpp", "topk_kernel.hpp", "libtopk.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "top_selection_two_amd", "csrc", name),
                  "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from committed counter runs, if still valid."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def time_oracle(x, k, budget_s=12.0, max_reps=3):
    """Median wall time of the single-threaded CPU oracle on x."""
    import oracle
    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps:
        t0 = time.perf_counter()
        oracle.topk(x, k)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    return statistics.median(times), len(times)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["bench", "counters"], default="bench")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grid", type=int, default=0,
                    help="stage-1 workgroups (0 = library default)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
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

    x = synth.workload(WORKLOAD)
    n = x.size
    xd = torch.from_numpy(x).to(dev)
    out = torch.empty(K, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.mode == "counters":
        # A plain copy of known size (calibrates the counters), then a few
        # top-k launches.
        src = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        for _ in range(5):
            ltk.topk(xd, K, out=out)
        torch.cuda.synchronize()
        print("counters mode: copy %d bytes read + %d written; 5 topk calls "
              "over n=%d" % (4 * n, 4 * n, n), flush=True)
        return

    # Correctness first (the oracle is the CPU reference; test-only code).
    import oracle
    got = ltk.topk(xd, K, out=out).cpu().numpy()
    want = oracle.topk(x, K)
    if not np.array_equal(got, want):
        print("MISMATCH against the oracle", got, want, file=sys.stderr)
        sys.exit(3)

    for _ in range(args.warmup):
        ltk.topk(xd, K, out=out)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        ltk.topk(xd, K, out=out)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    ms_per_step = wall * 1e3 / args.steps
    value = n * args.steps / wall

    algo_bytes = 4 * n + 4 * K
    achieved = algo_bytes / (avg_launch_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4),
        "traffic": measured_traffic(),
    }

    cpu = None
    if not args.no_cpu_baseline:
        t_med, reps = time_oracle(x, K)
        cpu = {
            "value": round(n / t_med, 1),
            "unit": "elements/s",
            "cores": 1,
            "kind": "oracle",
            "sample": "the full workload (1e8 int32, seed 3), top-20 by "
                      "copy + std::sort on one thread; median of %d run(s) "
                      "of %.2f s; host %s, %d logical CPUs"
                      % (reps, t_med, cpu_model(), os.cpu_count() or 0),
        }

    line = {
        "metric": METRIC,
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
        "config": {
            "workload": "top-20 of 1e8 int32, uniform over the full int32 "
                        "range (SplitMix64 seed 3), resident in HBM",
            "n": n,
            "k": K,
            "grid": ltk.grid_for(n),
            "kernel_ms_avg": round(avg_launch_ms, 5),
            "kernel_ms_min": round(min(launch_ms), 5),
            "hbm_gbps_per_step": round(algo_bytes / (ms_per_step * 1e-3) / 1e9,
                                       1),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
