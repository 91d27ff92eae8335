"""Benchmark of the fused SwiGLU + top-k weight + FP8/FP4 cast on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one launch of the fused kernel over one whole batch of the
workload (inputs resident in HBM).  The timed region is exactly K steps
bracketed by device synchronisations; per-launch durations come from HIP
events recorded on the launch stream.  Inputs and outputs rotate over
several buffer sets whose combined footprint is far above the 256 MB
Infinity Cache, so every launch streams from HBM.

Prints one JSON line on stdout.  The CPU baseline is the oracle, timed on a
bounded sample of the same workload's rows on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
KERNEL_SOURCE = os.path.join(ROOT, "moe_activation_bit_amd", "csrc", "tk_swiglu_cast.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def traffic_for(workload: str, launches_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, seed: int, rows: int):
    """The oracle on `rows` rows of the workload, split over host threads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from moe_activation_bit_amd import workloads as wl

    n = wl.num_rows(w, seed)
    rows = min(rows, n)
    x = wl.make_x(w, seed, rows=range(rows))
    wt = wl.make_w(w, seed)[:rows]
    fmt = 8 if w.fmt == "fp8" else 4
    sfmt = 0 if w.scale_fmt == "fp32" else 1
    threads = max(1, min(16, os.cpu_count() or 1, rows))
    spans = np.array_split(np.arange(rows), threads)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda s: oracle.swiglu_cast(x[s[0]:s[-1] + 1], wt[s[0]:s[-1] + 1], w.group_size,
                                                 w.clamp_limit, fmt, sfmt), [s for s in spans if len(s)]))
    dt = time.perf_counter() - t0
    return {
        "value": round(w.algorithmic_bytes(rows) / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {n} rows of {w.name} (seed {seed}); {dt:.2f} s wall, "
                  f"{rows / dt:.1f} rows/s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output buffer sets")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path "
            "(rows are independent; see the sharding notes). Run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch

    import moe_activation_bit_amd as tk
    from moe_activation_bit_amd import workloads as wl

    name = args.workload or wl.HEADLINE
    w = wl.WORKLOADS[name]
    n = wl.num_rows(w, args.seed)
    fmt = 8 if w.fmt == "fp8" else 4
    sfmt = tk.TK_SCALE_FP32 if w.scale_fmt == "fp32" else tk.TK_SCALE_UE8M0
    fn = tk.tk_swiglu_cast_fp8 if fmt == 8 else tk.tk_swiglu_cast_fp4
    clamp = math.inf if w.clamp_limit is None else w.clamp_limit
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    assert tk.tk_init(0) == tk.TkStatus.TK_OK

    log(f"[bench] workload {name}: rows {n}, hidden {w.hidden}, steps {args.steps}, warmup {args.warmup}")
    x_host = wl.make_x(w, args.seed)
    w_host = wl.make_w(w, args.seed)
    sets = []
    for _ in range(max(1, args.sets)):
        sets.append(dict(
            x=torch.from_numpy(x_host.view(np.int16)).to(dev),
            w=torch.from_numpy(w_host).to(dev),
            codes=torch.empty((n, w.code_bytes_per_row), dtype=torch.uint8, device=dev),
            scales=torch.empty((n, w.groups_per_row), dtype=torch.float32 if sfmt == 0 else torch.uint8, device=dev),
            count=torch.zeros(1, dtype=torch.int64, device=dev),
        ))
    del x_host
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    def step(i):
        s = sets[i % len(sets)]
        rc = fn(s["x"], s["w"], n, w.hidden, w.group_size, clamp, sfmt, s["codes"], s["scales"],
                s["count"] if w.clamp_limit is not None else None, sh)
        if rc != tk.TkStatus.TK_OK:
            raise RuntimeError(tk.tk_status_str(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    # Two HIP events on the launch stream bracket the K back-to-back launches
    # (events between launches would insert gaps of their own).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    log("[bench] timed region done")

    bytes_per_step = w.algorithmic_bytes(n)
    ms_per_step = elapsed / args.steps * 1e3
    value = bytes_per_step * args.steps / elapsed / 1e9
    avg_launch_s = gpu_s / args.steps
    achieved = bytes_per_step / avg_launch_s / 1e9
    traffic = traffic_for(name, bytes_per_step)

    out = {
        "metric": "fused SwiGLU+quant HBM GB/s (frac of peak) and rows/s at 1 MI355X",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": name, "rows": n, "hidden": w.hidden, "group_size": w.group_size,
                   "format": "e4m3" if fmt == 8 else "e2m1", "scale": w.scale_fmt, "clamp": w.clamp_limit,
                   "input": "bf16 [rows, 2*hidden]", "parallelism": "none (1 GPU)"},
        "rows_per_s": round(n * args.steps / elapsed, 1),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "swiglu_cast_kernel",
            "algorithmic_bytes_per_launch": bytes_per_step,
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
