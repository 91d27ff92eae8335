"""Benchmark of the fused SwiGLU + top-k weight + FP8/FP4 cast on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
python bench.py --kernel cast|topk|reduce|pos   (the next-row kernels, each on its own workload)
python bench.py --suite [--record FILE] [--baseline FILE]
    (every workload of every kernel, one JSON record per case; a case more
    than 15% slower than its committed baseline record is a regression and
    the exit code is 1)

One step = one launch of the kernel over one whole batch of the workload
(inputs resident in HBM).  The timed region is exactly K back-to-back steps
bracketed by device synchronisations and by two HIP events on the launch
stream (GPU time per launch = event time / K).  Inputs and outputs rotate
over several buffer sets whose combined footprint is far above the 256 MB
Infinity Cache, so every launch streams from HBM.

Prints one JSON line on stdout.  The CPU baseline is the oracle, timed on a
bounded sample of the same workload's rows on the host's cores.

HBM traffic (roofline.traffic) comes from two rocprofv3 counter runs of
`bench.py [--kernel K] --steps 5 --warmup 1 --no-cpu-baseline --copy-calibration`,
one with `--pmc FETCH_SIZE`, one with `--pmc WRITE_SIZE`; `bench.py [--kernel K]
--summarize-pmc FETCH.csv WRITE.csv` scales that kernel's per-dispatch counters
by what the same counters read for a plain elementwise copy of known size and
writes profiles/traffic_<workload>.json (tagged with the kernel source digest;
a stale record is ignored).  The gating's line also carries valu_issue: VALU
instructions per launch from a `--pmc SQ_INSTS_VALU SQ_WAVES ...` run, recorded
by `bench.py --kernel topk --summarize-valu PMC.csv` in
profiles/valu_<workload>.json, against the chip's VALU issue rate.
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

# Each timed kernel: the sources its counters depend on, how its name reads
# in a rocprofv3 trace, and the name the bench line gives it.
KERNELS = {
    "fused": (("tk_swiglu_cast.hip", "tk_quant.h"), r"\bswiglu_cast_kernel<", "swiglu_cast_kernel"),
    "cast": (("tk_cast.hip", "tk_quant.h"), r"\bcast_kernel<", "cast_kernel"),
    "reduce": (("tk_reduce.hip",), r"\bmoe_reduce_kernel<", "moe_reduce_kernel"),
    # (three launches per call; the line names the last, which writes the map)
    "pos": (("tk_pos.hip",), r"\bpos_(?:count|scan|write)_kernel", "pos_write_kernel"),
    # (topk_row_kernel serves the gating workload's shape: 256 experts, 8
    # groups keep 4, top-8)
    "topk": (("tk_topk.hip",), r"\btopk_(?:pair_|quad_|row_)?kernel<", "topk_row_kernel"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text with comments removed and whitespace collapsed, so that a
    comment edit leaves the digest (and the counters tied to it) unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(kernel: str = "fused") -> str:
    h = hashlib.sha256()
    for f in KERNELS[kernel][0]:
        h.update(_code_only(open(os.path.join(ROOT, "moe_activation_bit_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str = "fused"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes


def copy_calibration(torch, dev):
    """A plain elementwise copy of known size (read COPY_CAL_BYTES, write
    COPY_CAL_BYTES) for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _pmc_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def aux_workload(kernel: str, wl, seed: int):
    """(workload name, algorithmic bytes per launch) of a bench mode, from the
    host-side description alone."""
    if kernel == "fused":
        raise ValueError("the fused kernel's workloads are in workloads.WORKLOADS")
    if kernel == "cast":
        n, hidden, group = 2 * CAST_TOKENS, CAST_HIDDEN, CAST_GROUP
        return (f"cast_bf16_e4m3_g{group}_ue8m0_n{n}_h{hidden}",
                n * (2 * hidden + hidden + hidden // group))
    if kernel == "reduce":
        r = wl.REDUCE_WORKLOADS[wl.REDUCE_HEADLINE]
        pos, _, _, _ = wl.make_routing(r, seed)
        return r.name, r.algorithmic_bytes(pos)
    if kernel == "pos":
        T, E, k = POS_SHAPE
        return f"topk_to_pos_t{T}_k{k}_e{E}", T * k * 8 + (E + 1) * 4
    T, E, k, ng, tg = TOPK_SHAPE
    return f"topk_gate_t{T}_e{E}_g{ng}_keep{tg}_top{k}", T * (4 * E + 8 * k)


def summarize_pmc(fetch_csv: str, write_csv: str, kernel: str, workload: str, seed: int):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of one kernel, scaled by the
    calibration copy's readings; writes profiles/traffic_<workload>.json."""
    import re

    from moe_activation_bit_amd import workloads as wl

    if kernel == "fused":
        w = wl.workload(workload)
        algo = w.algorithmic_bytes(wl.num_rows(w, seed))
    else:
        workload, algo = aux_workload(kernel, wl, seed)
    pat = re.compile(KERNELS[kernel][1])

    def per_dispatch(rows, counter, pick):
        vals = [float(r["Counter_Value"]) for r in rows
                if r.get("Counter_Name") == counter and pick(r.get("Kernel_Name", ""))]
        return sum(vals) / len(vals) if vals else None, len(vals)

    mine = lambda k: bool(pat.search(k))
    copy = lambda k: "MulFunctor" in k  # torch.mul(src, 1.0, out=dst): the calibration copy
    f_rows, w_rows = _pmc_rows(fetch_csv), _pmc_rows(write_csv)
    f_kib, nf = per_dispatch(f_rows, "FETCH_SIZE", mine)
    w_kib, nw = per_dispatch(w_rows, "WRITE_SIZE", mine)
    cf_kib, ncf = per_dispatch(f_rows, "FETCH_SIZE", copy)
    cw_kib, ncw = per_dispatch(w_rows, "WRITE_SIZE", copy)
    if None in (f_kib, w_kib, cf_kib, cw_kib):
        raise SystemExit("counter rows missing: kernel %s/%s copy %s/%s" % (nf, nw, ncf, ncw))
    fetch_scale = (COPY_CAL_BYTES / 1024.0) / cf_kib
    write_scale = (COPY_CAL_BYTES / 1024.0) / cw_kib
    fetch_bytes = f_kib * 1024.0 * fetch_scale
    write_bytes = w_kib * 1024.0 * write_scale
    rec = {
        "workload": workload,
        "kernel": kernel,
        "kernel_source_sha256_16": kernel_source_digest(kernel),
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
        "copy_fetch_kib_per_dispatch": cf_kib, "copy_write_kib_per_dispatch": cw_kib,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_bytes_per_launch": round(fetch_bytes + write_bytes),
        "algorithmic_bytes_per_launch": algo,
        "dispatches": {"kernel_fetch": nf, "kernel_write": nw, "copy_fetch": ncf, "copy_write": ncw},
    }
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


# VALU issue peak of the chip: 256 CUs x 4 SIMDs, one wave64 VALU instruction
# per SIMD every 4 cycles, 2.4 GHz
VALU_PEAK_INSTS_PER_S = 256 * 4 * 2.4e9 / 4


def summarize_valu(csv_path: str, kernel: str, seed: int):
    """Per-dispatch SQ_INSTS_VALU / SQ_WAVES of one kernel from a rocprofv3
    counter run; writes profiles/valu_<workload>.json (tagged with the kernel
    source digest, like the traffic records)."""
    import re

    from moe_activation_bit_amd import workloads as wl

    workload, _ = aux_workload(kernel, wl, seed)
    pat = re.compile(KERNELS[kernel][1])
    vals = {}
    for r in _pmc_rows(csv_path):
        if pat.search(r.get("Kernel_Name", "")) and r.get("Counter_Name") in ("SQ_INSTS_VALU", "SQ_WAVES"):
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if set(vals) != {"SQ_INSTS_VALU", "SQ_WAVES"}:
        raise SystemExit("counter rows missing: need SQ_INSTS_VALU and SQ_WAVES")
    rec = {"workload": workload, "kernel": kernel, "kernel_source_sha256_16": kernel_source_digest(kernel),
           "valu_insts_per_dispatch": sum(vals["SQ_INSTS_VALU"]) / len(vals["SQ_INSTS_VALU"]),
           "waves_per_dispatch": sum(vals["SQ_WAVES"]) / len(vals["SQ_WAVES"]),
           "dispatches": len(vals["SQ_INSTS_VALU"])}
    with open(os.path.join(ROOT, "profiles", f"valu_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def valu_for(workload: str, kernel: str):
    """VALU instructions per launch from the committed counter record, if it
    was taken on the current kernel code; else None."""
    path = os.path.join(ROOT, "profiles", f"valu_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_digest(kernel):
        return None
    return rec.get("valu_insts_per_dispatch")


INFINITY_CACHE_BYTES = 256 * 2**20  # MI355X last-level (Infinity) cache
LAUNCH_BOUND_US = 5.0  # below this HBM time per launch, dispatch and ramp dominate


def regime(bytes_per_launch, sets, avg_launch_s, compute_us=0.0):
    """Labels a line by what bounds it.  `cache` is "hot" when every rotating
    buffer set together fits the Infinity Cache (the timed launches then read
    from cache, not HBM), else "streamed".  `launch_bound` is set when the
    algorithmic bytes would take under LAUNCH_BOUND_US at HBM peak and the
    launch's own issue bound (`compute_us`, e.g. its VALU instructions at the
    chip's issue rate) is under it too: then the roofline fraction measures
    launch latency, and `us_per_call` is the number to read."""
    footprint = bytes_per_launch * sets
    hbm_us = bytes_per_launch / (HBM_PEAK_GBS * 1e9) * 1e6
    return {
        "cache": "hot" if footprint <= INFINITY_CACHE_BYTES else "streamed",
        "rotating_footprint_bytes": footprint,
        "launch_bound": max(hbm_us, compute_us) < LAUNCH_BOUND_US,
        "hbm_peak_us": round(hbm_us, 3),
        "us_per_call": round(avg_launch_s * 1e6, 3),
    }


def unfused_path(torch, tk, dev, w, n, fmt, sfmt, clamp, sets, reps, stream, fused_s):
    """The unfused reference of the same step (swiglu_forward writes fp32 y to
    HBM, then the stand-alone cast reads it), timed like the fused step; its
    effective bandwidth counts the same algorithmic bytes."""
    y = [torch.empty((n, w.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
    cast = tk.tk_cast_fp8 if fmt == 8 else tk.tk_cast_fp4
    sh = int(stream.cuda_stream)

    def step(i):
        s = sets[i % len(sets)]
        yy = y[i % 2]
        rc = tk.tk_swiglu_forward(s["x"], s["w"], n, w.hidden, clamp, yy,
                                  s["count"] if w.clamp_limit is not None else None, sh)
        assert rc == tk.TkStatus.TK_OK, rc
        rc = cast(yy, tk.TK_DTYPE_FP32, n, w.hidden, w.group_size, sfmt, s["codes"], s["scales"], sh)
        assert rc == tk.TkStatus.TK_OK, rc

    for i in range(3):
        step(i)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(reps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) / 1e3 / reps
    del y
    torch.cuda.empty_cache()
    return {"us_per_step": round(t * 1e6, 3),
            "effective_GBs": round(w.algorithmic_bytes(n) / t / 1e9, 1),
            "hbm_bytes_per_step": w.algorithmic_bytes(n) + 2 * 4 * w.hidden * n,
            "fused_speedup": round(t / fused_s, 3),
            "kernels": "tk_swiglu_forward (fp32 y out) + tk_cast (fp32 y in)"}


# The 4:1 probe's matrix: cache-policy bits of the loads and of the stores
# (0: none, 2: nt, 16: sc1, 17: sc0 sc1) x grid (steps per unit, workgroups
# per CU; 0 = non-persistent, one unit per wave).
PROBE_POLICIES = (0, 2, 16, 17)
PROBE_GRIDS = ((1, 0), (4, 0), (4, 2))
POLICY_NAMES = {0: "plain", 2: "nt", 16: "sc1", 17: "sc0sc1"}


def stream_ceiling(torch, dev, rows: int, hidden: int, reps: int = 10, rounds: int = 3):
    """GB/s of plain streaming kernels moving the workload's bytes with no
    arithmetic.  The ceiling is the fastest of the 4:1 probe's matrix (the
    fused step's own layout: gate and up halves of a packed bf16 row in, one
    byte per column out) over load policy x store policy x grid, each combination
    timed `rounds` times interleaved (median kept); a plain read-only stream
    over the same input is reported beside it."""
    import ctypes
    import statistics
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_activation_bit_amd", "libstreamceil.so"))
    lib.stream_probe_4to1.restype = ctypes.c_int
    lib.stream_probe_4to1.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_uint32, ctypes.c_void_p]
    lib.stream_read_only.restype = ctypes.c_int
    lib.stream_read_only.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    # the probe needs whole 2048-column rows: the same bytes laid out that way
    ph = 2048
    prow = max(1, (rows * hidden + ph - 1) // ph)
    in_bytes, out_bytes = prow * 4 * ph, prow * ph
    nbytes = in_bytes + out_bytes
    sets = 2
    ins = [torch.ones(in_bytes // 4, dtype=torch.int32, device=dev) for _ in range(sets)]
    outs = [torch.empty(out_bytes // 4, dtype=torch.int32, device=dev) for _ in range(sets)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    def timed(fn):
        for i in range(3):
            fn(i)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / reps

    def probe(lp, sp, spu, bpc):
        def fn(i):
            assert lib.stream_probe_4to1(ins[i % sets].data_ptr(), outs[i % sets].data_ptr(), prow, ph, lp, sp,
                                         spu, bpc, cus, sh) == 0
        return fn

    combos = [(lp, sp, spu, bpc) for lp in PROBE_POLICIES for sp in PROBE_POLICIES for spu, bpc in PROBE_GRIDS]
    times = {c: [] for c in combos}
    for _ in range(rounds):
        for c in combos:
            times[c].append(timed(probe(*c)))

    def ro(i):
        assert lib.stream_read_only(ins[i % sets].data_ptr(), in_bytes, sink.data_ptr(), sh) == 0

    ro_s = timed(ro)
    gbs = {c: nbytes / statistics.median(t) / 1e9 for c, t in times.items()}
    best = max(gbs, key=gbs.get)

    def label(c):
        lp, sp, spu, bpc = c
        grid = f"persistent{bpc}x{spu}" if bpc else f"nonpersistent{spu}"
        return f"load={POLICY_NAMES[lp]},store={POLICY_NAMES[sp]},grid={grid}"

    res = {"read4_write1_GBs": round(gbs[best], 1),
           "best": label(best),
           "read_only_GBs": round(in_bytes / ro_s / 1e9, 1),
           "bytes_per_launch": nbytes,
           "matrix_GBs": {label(c): round(v, 1) for c, v in sorted(gbs.items(), key=lambda kv: -kv[1])},
           "kernel": f"probe_4to1_kernel: packed bf16 [{prow}, {2 * ph}] in as gate/up halves, "
                     f"[{prow}, {ph}] bytes out; median of {rounds} interleaved rounds of {reps} launches"}
    del ins, outs
    torch.cuda.empty_cache()
    return res


# The next-row kernels' read:write mixes for the plain-stream probe: 16-byte
# vectors read and bytes written per probe thread (the cast: 16 bytes of bf16
# in, 8 code bytes out; the gating: 64 bytes of scores in, 4 bytes of indices
# and weights out).  The scale bytes the cast also writes (1/256 of its
# traffic) are left out.
STREAM_MIX = {"cast": (1, 8), "topk": (4, 4)}


def stream_mix(torch, dev, in_bytes: int, rv: int, wb: int, sets: int, reps: int = 200, rounds: int = 3):
    """GB/s of a plain non-temporal stream with a kernel's read:write mix:
    in_bytes read and in_bytes * wb / (16 * rv) written per launch, no
    arithmetic, over `sets` rotating buffer sets like the kernel's own line;
    median of `rounds` rounds of `reps` launches."""
    import ctypes
    import statistics
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_activation_bit_amd", "libstreamceil.so"))
    lib.stream_read_n_write.restype = ctypes.c_int
    lib.stream_read_n_write.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_void_p]
    n = in_bytes // (16 * rv)
    assert n * 16 * rv == in_bytes and n > 0
    out_bytes = n * wb
    ins = [torch.ones(in_bytes // 4, dtype=torch.int32, device=dev) for _ in range(sets)]
    outs = [torch.empty((out_bytes + 3) // 4, dtype=torch.int32, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    def launch(i):
        assert lib.stream_read_n_write(ins[i % sets].data_ptr(), outs[i % sets].data_ptr(), n, rv, wb, sh) == 0

    for i in range(max(50, sets)):
        launch(i)
    times = []
    for _ in range(rounds):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            launch(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3 / reps)
    t = statistics.median(times)
    del ins, outs
    torch.cuda.empty_cache()
    return {"stream_GBs": round((in_bytes + out_bytes) / t / 1e9, 1), "us_per_launch": round(t * 1e6, 3),
            "bytes_per_launch": in_bytes + out_bytes,
            "kernel": f"read_n_write_kernel<{rv}, {wb}>: {n} threads, {16 * rv} bytes read and {wb} written "
                      f"each, non-temporal, non-persistent; {sets} rotating sets; median of {rounds} rounds of "
                      f"{reps} launches"}


def cpu_baseline(w, seed: int, rows: int, single_rows: int = 1024):
    """The oracle on `rows` rows of the workload, split over host threads (the
    reported value), and on `single_rows` of them on one thread."""
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

    def run(a, b):
        oracle.swiglu_cast(x[a:b], wt[a:b], w.group_size, w.clamp_limit, fmt, sfmt)

    threads = max(1, min(16, os.cpu_count() or 1, rows))
    spans = [s for s in np.array_split(np.arange(rows), threads) if len(s)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:  # ctypes calls release the GIL
        list(ex.map(lambda s: run(int(s[0]), int(s[-1]) + 1), spans))
    dt = time.perf_counter() - t0
    r1 = min(single_rows, rows)
    t1 = time.perf_counter()
    run(0, r1)
    dt1 = time.perf_counter() - t1
    return {
        "value": round(w.algorithmic_bytes(rows) / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {n} rows of {w.name} (seed {seed}); {dt:.2f} s wall on {threads} threads "
                  f"({dt * threads:.1f} thread-s), {rows / dt:.1f} rows/s",
        "single_thread": {"value": round(w.algorithmic_bytes(r1) / dt1 / 1e9, 6), "unit": "GB/s",
                          "rows": r1, "seconds": round(dt1, 3)},
        "rows_per_s": round(rows / dt, 1),
        "host": host_cpu(),
    }


def host_cpu() -> dict:
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"logical_cpus": os.cpu_count(), "cpu_model": model}


def flushed_reps(torch, step, nbytes: int, reps: int = 30, warm: int = 3):
    """3 warm-up launches, then `reps` launches each preceded by a 1 GiB write
    and read of a scratch buffer (the 256 MB Infinity Cache holds none of the
    inputs afterwards) and bracketed by two events; median, min and max."""
    import statistics

    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for i in range(warm):
        step(i)
    times = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        flush.max()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        step(i)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3)
    del flush
    med = statistics.median(times)
    return {"reps": reps, "median_us": round(med * 1e6, 3), "min_us": round(min(times) * 1e6, 3),
            "max_us": round(max(times) * 1e6, 3), "GBs_median": round(nbytes / med / 1e9, 3),
            "frac_median": round(nbytes / med / 1e9 / HBM_PEAK_GBS, 4)}


def graph_replay(torch, step, steps: int, nbytes: int):
    """The same K launches captured once in a HIP graph (torch.cuda.graph) and
    replayed: GPU time per launch without host launch overhead, which is what
    bounds the small, latency-bound workloads."""
    here = lambda: int(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            step(i, here())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = here()  # the capture stream
        for i in range(steps):
            step(i, cap)
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    per = ev0.elapsed_time(ev1) / 1e3 / steps
    return {"launches_per_graph": steps, "us_per_launch": round(per * 1e6, 3),
            "GBs": round(nbytes / per / 1e9, 3)}


def _timed(torch, stream, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ev0.elapsed_time(ev1) / 1e3


CAST_TOKENS, CAST_HIDDEN, CAST_GROUP = 32768, 2048, 128
TOPK_SHAPE = (16384, 256, 8, 8, 4)  # tokens, experts, k, groups, groups kept
POS_SHAPE = (16384, 256, 8)  # tokens, experts, k: the gating workload's indices


def aux_setup(kernel, torch, np, tk, wl, seed, sets, dev, sh):
    """Device buffers and the launch closure of one next-row kernel on its own
    workload: the stand-alone cast (bf16 [65536, 2048] -> E4M3, groups of 128,
    UE8M0), the top-k gating (16384 tokens x 256 experts, 8 groups, keep 4,
    top-8, normalised) or the weighted top-k reduce (4096 tokens x top-8,
    hidden 7168, bf16 rows gathered through the position map).  Returns
    (workload name, algorithmic bytes per launch, step(i), metric, config, rows)."""
    name, nbytes = aux_workload(kernel, wl, seed)
    if kernel == "cast":
        n, hidden, group = CAST_TOKENS, CAST_HIDDEN, CAST_GROUP
        w = wl.Workload(name, n, hidden, 2.0, "fp8", group, "ue8m0", None, "uniform")
        xh = wl.make_x(w, seed)  # [n, 2*hidden] bf16 N(0,2) samples, read as [2n, hidden] rows
        assert xh.size == 2 * n * hidden
        n2 = 2 * n
        xs = [torch.from_numpy(xh.view(np.int16)).to(dev) for _ in range(sets)]
        cs = [torch.empty((n2, hidden), dtype=torch.uint8, device=dev) for _ in range(sets)]
        ss = [torch.empty((n2, hidden // group), dtype=torch.uint8, device=dev) for _ in range(sets)]
        del xh

        def step(i, stream_handle=sh):
            k = i % sets
            rc = tk.tk_cast_fp8(xs[k], tk.TK_DTYPE_BF16, n2, hidden, group, tk.TK_SCALE_UE8M0, cs[k], ss[k],
                                stream_handle)
            assert rc == tk.TkStatus.TK_OK, rc
        metric = "stand-alone bf16->FP8 cast HBM GB/s (frac of peak) at 1 MI355X"
        config = {"workload": name, "rows": n2, "hidden": hidden, "group_size": group, "format": "e4m3",
                  "scale": "ue8m0", "input": "bf16 [rows, hidden]"}
        rows = n2
    elif kernel == "reduce":
        r = wl.REDUCE_WORKLOADS[wl.REDUCE_HEADLINE]
        pos, wts, rsc, n_rows = wl.make_routing(r, seed)
        xh = wl.make_expert_rows(r, seed, n_rows)
        xs = [torch.from_numpy(xh.view(np.int16)).to(dev) for _ in range(sets)]
        del xh
        pd, wd, rd = (torch.from_numpy(pos).to(dev), torch.from_numpy(wts).to(dev), torch.from_numpy(rsc).to(dev))
        outs = [torch.empty((r.tokens, r.hidden), dtype=torch.bfloat16, device=dev) for _ in range(sets)]

        def step(i, stream_handle=sh):
            j = i % sets
            rc = tk.tk_moe_reduce(xs[j], rd, pd, wd, r.global_scale, r.tokens, r.k, r.hidden, n_rows,
                                  tk.TK_DTYPE_BF16, outs[j], stream_handle)
            assert rc == tk.TkStatus.TK_OK, rc
        metric = "weighted top-k MoE reduce HBM GB/s (frac of peak) at 1 MI355X"
        config = {"workload": name, "tokens": r.tokens, "k": r.k, "experts": r.experts, "hidden": r.hidden,
                  "n_rows": n_rows, "row_scale": r.row_scale, "global_scale": r.global_scale, "out": "bf16",
                  "layout": "rows grouped by expert, tokens in order within an expert"}
        rows = r.tokens
    elif kernel == "pos":
        T, E, k = POS_SHAPE
        # k distinct experts per token, drawn from the seeded uniform stream
        u = wl.uniform(wl.stream_key("topk_to_pos", seed, "experts"), 0, T * E).reshape(T, E)
        ih = np.ascontiguousarray(np.argsort(u, axis=1)[:, :k].astype(np.int32))
        ids = [torch.from_numpy(ih).to(dev) for _ in range(sets)]
        ps = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(sets)]
        offs = [torch.empty((E + 1,), dtype=torch.int32, device=dev) for _ in range(sets)]

        def step(i, stream_handle=sh):
            j = i % sets
            rc = tk.tk_topk_to_pos(ids[j], T, k, E, ps[j], offs[j], stream_handle)
            assert rc == tk.TkStatus.TK_OK, rc
        metric = "token/top-k -> expert-row map tokens/s and HBM GB/s at 1 MI355X"
        config = {"workload": name, "tokens": T, "experts": E, "k": k,
                  "routing": "k distinct experts per token, uniform", "launches_per_call": 3}
        rows = T
    else:
        T, E, k, ng, tg = TOPK_SHAPE
        key = wl.stream_key("topk_gate", seed, "scores")
        sh_ = wl.uniform(key, 0, T * E).reshape(T, E).astype(np.float32)
        sc = [torch.from_numpy(sh_).to(dev) for _ in range(sets)]
        idx = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(sets)]
        wt = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(sets)]

        def step(i, stream_handle=sh):
            j = i % sets
            rc = tk.tk_topk_gate(sc[j], T, E, k, ng, tg, 1, idx[j], wt[j], stream_handle)
            assert rc == tk.TkStatus.TK_OK, rc
        metric = "deterministic top-k gating tokens/s and HBM GB/s at 1 MI355X"
        config = {"workload": name, "tokens": T, "experts": E, "k": k, "n_group": ng, "topk_group": tg,
                  "normalise": True, "scores": "U(0,1) fp32"}
        rows = T
    return name, nbytes, step, metric, config, rows


def aux_sets(kernel, requested=None):
    """Rotating buffer sets of a next-row line: 4, or 32 for the gating, whose
    17.8 MB per launch would otherwise stay in the Infinity Cache (32 sets,
    570 MB, make it read from HBM like the other lines)."""
    return max(1, requested if requested is not None else (32 if kernel == "topk" else 4))


def bench_aux(args, torch, np, tk, wl):
    """The next-row kernels on their own workloads, one JSON line like the
    headline's (see aux_setup for the workloads)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    assert tk.tk_init(0) == tk.TkStatus.TK_OK
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    sets = aux_sets(args.kernel, args.sets)
    if args.copy_calibration:
        copy_calibration(torch, dev)
    name, nbytes, step, metric, config, rows = aux_setup(args.kernel, torch, np, tk, wl, args.seed, sets, dev, sh)
    kernel = KERNELS[args.kernel][2]
    wall, gpu = _timed(torch, stream, step, args.steps, args.warmup)
    avg = gpu / args.steps
    achieved = nbytes / avg / 1e9
    out = {"metric": metric, "value": round(nbytes * args.steps / wall / 1e9, 3), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp32", "data": "synthetic", "config": config,
           "rows_per_s": round(rows * args.steps / wall, 1),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(name, args.kernel),
                        "kernel": kernel, "algorithmic_bytes_per_launch": nbytes,
                        "avg_launch_us": round(avg * 1e6, 3)},
           "regime": regime(nbytes, sets, avg),
           "cpu_baseline": None}
    if args.kernel in STREAM_MIX and not args.no_ceiling:
        # what a plain stream with the kernel's own read:write mix reaches
        rv, wb = STREAM_MIX[args.kernel]
        in_bytes = (CAST_TOKENS * 2 * CAST_HIDDEN * 2 if args.kernel == "cast"
                    else TOPK_SHAPE[0] * TOPK_SHAPE[1] * 4)
        ceil = stream_mix(torch, dev, in_bytes, rv, wb, sets)
        out["roofline"]["measured_ceiling"] = ceil
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["stream_GBs"], 4)
    if args.kernel == "topk":
        # the gating's VALU instructions per launch (counter record) against
        # the chip's issue rate, beside its bytes
        v = valu_for(name, "topk")
        out["valu_issue"] = None if v is None else {
            "insts_per_launch": round(v), "achieved": round(v / avg / 1e9, 2), "peak": VALU_PEAK_INSTS_PER_S / 1e9,
            "unit": "G wave64 VALU instructions/s", "frac": round(v / avg / VALU_PEAK_INSTS_PER_S, 4)}
        if v is not None:
            out["regime"] = regime(nbytes, sets, avg, v / VALU_PEAK_INSTS_PER_S * 1e6)
    print(json.dumps(out), flush=True)


def fused_setup(torch, np, tk, wl, name, seed, nsets, dev, sh):
    """Device buffers (nsets rotating sets of x, topk_weight, codes, scales and
    the clamp counter) and the launch closure step(i[, stream]) of one fused
    workload.  Returns (workload, rows, fmt, scale fmt, clamp limit, sets, step)."""
    w = wl.workload(name)
    n = wl.num_rows(w, seed)
    fmt = 8 if w.fmt == "fp8" else 4
    sfmt = tk.TK_SCALE_FP32 if w.scale_fmt == "fp32" else tk.TK_SCALE_UE8M0
    fn = tk.tk_swiglu_cast_fp8 if fmt == 8 else tk.tk_swiglu_cast_fp4
    clamp = math.inf if w.clamp_limit is None else w.clamp_limit
    x_host = wl.make_x(w, seed)
    w_host = wl.make_w(w, seed)
    sets = []
    for _ in range(max(1, nsets)):
        sets.append(dict(
            x=torch.from_numpy(x_host.view(np.int16)).to(dev),
            w=torch.from_numpy(w_host).to(dev),
            codes=torch.empty((n, w.code_bytes_per_row), dtype=torch.uint8, device=dev),
            scales=torch.empty((n, w.groups_per_row), dtype=torch.float32 if sfmt == 0 else torch.uint8, device=dev),
            count=torch.zeros(1, dtype=torch.int64, device=dev),
        ))
    del x_host

    def step(i, stream_handle=sh):
        s = sets[i % len(sets)]
        rc = fn(s["x"], s["w"], n, w.hidden, w.group_size, clamp, sfmt, s["codes"], s["scales"],
                s["count"] if w.clamp_limit is not None else None, stream_handle)
        if rc != tk.TkStatus.TK_OK:
            raise RuntimeError(tk.tk_status_str(rc))
    return w, n, fmt, sfmt, clamp, sets, step


# The benchmark suite: every workload of the fused kernel and the next-row
# kernels' lines, one record per case, compared with a committed baseline by
# the regression rule of TileKernels' benchmark plugin ("TileKernels从入门到精通"
# ch.5, "铁血防线"): a case regresses when its time exceeds the baseline's by
# more than the threshold (15% there).
BASELINES = os.path.join(ROOT, "profiles", "bench_baselines.jsonl")
REGRESSION_THRESHOLD = 0.15
SUITE_AUX = ("cast", "reduce", "topk", "pos")
SUITE_OPS = {"fused": "swiglu_cast", "cast": "cast", "reduce": "moe_reduce", "topk": "topk_gate",
             "pos": "topk_to_pos"}


def case_key(kernel: str, params: dict) -> str:
    """Record key in the pages' shape, op/fwd[k=v,...], sorted by parameter name."""
    inner = ",".join(f"{k}={params[k]}" for k in sorted(params))
    return f"{SUITE_OPS[kernel]}/fwd[{inner}]"


def compare_records(records, baseline, threshold=REGRESSION_THRESHOLD):
    """Each record against the baseline record of the same key.  Returns
    [(key, time_us, baseline_us or None, ratio or None, status)] with status
    "ok", "REGRESSION" (time / baseline > 1 + threshold), "new" (no baseline)
    and, for baseline keys this run did not measure, "missing"."""
    base = {b["key"]: b for b in baseline}
    out = []
    for r in records:
        b = base.get(r["key"])
        if b is None:
            out.append((r["key"], r["time_us"], None, None, "new"))
            continue
        ratio = r["time_us"] / b["time_us"]
        out.append((r["key"], r["time_us"], b["time_us"], ratio, "REGRESSION" if ratio > 1.0 + threshold else "ok"))
    seen = {r["key"] for r in records}
    out += [(k, None, b["time_us"], None, "missing") for k, b in base.items() if k not in seen]
    return out


def read_records(path):
    with open(path) as fh:
        return [json.loads(line) for line in fh if line.strip()]


def run_suite(args, torch, np, tk, wl):
    """Times every case (W warm-up then K back-to-back launches between two
    HIP events, as the headline line; launch-bound cases by the same K
    launches replayed from one HIP graph), prints one JSON record per case,
    optionally writes them to --record, and compares them with the baseline
    file; returns the process exit code (1 when a case regressed)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    assert tk.tk_init(0) == tk.TkStatus.TK_OK
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    cases = [("fused", name) for name in wl.WORKLOADS] + [(k, None) for k in SUITE_AUX]
    records = []
    for kernel, name in cases:
        if kernel == "fused":
            nsets = args.sets if args.sets is not None else 4
            w, n, fmt, _, _, sets, step = fused_setup(torch, np, tk, wl, name, args.seed, nsets, dev, sh)
            nbytes = w.algorithmic_bytes(n)
            params = {"workload": name, "num_tokens": n, "hidden": w.hidden, "group_size": w.group_size,
                      "fmt": "e4m3" if fmt == 8 else "e2m1", "scale": w.scale_fmt, "seed": args.seed}
            del sets
        else:
            nsets = aux_sets(kernel, args.sets)
            name, nbytes, step, _, _, _ = aux_setup(kernel, torch, np, tk, wl, args.seed, nsets, dev, sh)
            params = {"workload": name, "seed": args.seed}
        log(f"[suite] {kernel} {name} ...")
        _, gpu = _timed(torch, stream, step, args.steps, args.warmup)
        avg = gpu / args.steps
        v = valu_for(name, kernel) if kernel == "topk" else None
        reg = regime(nbytes, nsets, avg, 0.0 if v is None else v / VALU_PEAK_INSTS_PER_S * 1e6)
        timing = "events"
        if reg["launch_bound"]:
            # eager back-to-back launches of a few microseconds measure the host's
            # launch issue; the launches replayed from one HIP graph measure the GPU
            avg = graph_replay(torch, step, args.steps, nbytes)["us_per_launch"] / 1e6
            timing = "graph"
        rec = {"key": case_key(kernel, params), "kernel": KERNELS[kernel][2],
               "operation": "fwd", "params": params, "time_us": round(avg * 1e6, 3), "timing": timing,
               "bandwidth_gbs": round(nbytes / avg / 1e9, 1), "frac_of_peak": round(nbytes / avg / 1e9 / HBM_PEAK_GBS, 4),
               "regime": reg}
        records.append(rec)
        print(json.dumps(rec), flush=True)
        del step
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.record:
        with open(args.record, "w") as fh:
            for r in records:
                fh.write(json.dumps(r) + "\n")
    if not args.baseline or args.baseline == "none" or not os.path.exists(args.baseline):
        log("[suite] no baseline to compare with")
        return 0
    rows = compare_records(records, read_records(args.baseline), args.threshold)
    log(f"[suite] against {os.path.relpath(args.baseline, ROOT)} (regression: > {args.threshold:.0%} slower)")
    for key, t, b, ratio, status in rows:
        tt = "-" if t is None else f"{t:.2f}"
        bb = "-" if b is None else f"{b:.2f}"
        rr = "-" if ratio is None else f"{ratio:.3f}"
        log(f"  {status:<10} {tt:>9} us  baseline {bb:>9} us  ratio {rr:>6}  {key}")
    return 1 if any(r[4] == "REGRESSION" for r in rows) else 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 1000 warm-up launches (~60 ms of GPU work on the default workload): after
    # the seconds of idle host-side set-up the GPU needs that long to reach its
    # steady operating point (20 warm-up launches measured 61.7 us, 200 57.2,
    # 1000 56.6 on the default workload)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=None,
                    help="rotating input/output buffer sets (default 4; 32 for --kernel topk)")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-ceiling measurement")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused two-kernel comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain elementwise copy of known size first (for counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-valu", metavar="PMC_CSV",
                    help="record SQ_INSTS_VALU / SQ_WAVES per dispatch of --kernel topk from a counter run")
    ap.add_argument("--no-flushed", action="store_true",
                    help="skip the 30 single launches after a 1 GiB cache flush each (protocol_flush30)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the K launches captured in one HIP graph (reported as graph_replay)")
    ap.add_argument("--kernel", choices=["fused", "cast", "topk", "reduce", "pos"], default="fused",
                    help="fused (default): the fused SwiGLU + cast; cast: the stand-alone cast; topk: the gating; "
                         "reduce: the weighted top-k reduce; pos: the token/top-k -> expert-row map")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload of every kernel, one JSON record per case, and compare with "
                         "--baseline (exit code 1 when a case is more than --threshold slower)")
    ap.add_argument("--baseline", default=BASELINES,
                    help="baseline records for --suite ('none' to skip the comparison)")
    ap.add_argument("--record", default=None, help="write --suite's records to this JSONL file")
    ap.add_argument("--threshold", type=float, default=REGRESSION_THRESHOLD)
    args = ap.parse_args()

    if args.summarize_valu:
        summarize_valu(args.summarize_valu, args.kernel, args.seed)
        return
    if args.summarize_pmc:
        from moe_activation_bit_amd import workloads as wl
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.kernel, args.workload or wl.HEADLINE,
                      args.seed)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(rows are independent; see the sharding notes). Run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch

    import moe_activation_bit_amd as tk
    from moe_activation_bit_amd import workloads as wl

    if args.suite:
        sys.exit(run_suite(args, torch, np, tk, wl))
    if args.kernel != "fused":
        return bench_aux(args, torch, np, tk, wl)

    name = args.workload or wl.HEADLINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    assert tk.tk_init(0) == tk.TkStatus.TK_OK
    if args.copy_calibration:
        copy_calibration(torch, dev)
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    w, n, fmt, sfmt, clamp, sets, step = fused_setup(torch, np, tk, wl, name, args.seed,
                                                     args.sets if args.sets is not None else 4, dev, sh)
    log(f"[bench] workload {name}: rows {n}, hidden {w.hidden}, steps {args.steps}, warmup {args.warmup}")

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
    traffic = traffic_for(name, "fused")

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
        "regime": regime(bytes_per_step, len(sets), avg_launch_s),
        "cpu_baseline": None,
    }
    if not args.no_flushed:
        log("[bench] 30 flushed reps ...")
        out["protocol_flush30"] = flushed_reps(torch, step, bytes_per_step)
    if args.graph:
        log("[bench] graph replay ...")
        out["graph_replay"] = graph_replay(torch, step, args.steps, bytes_per_step)
    if not args.no_unfused:
        log("[bench] unfused two-kernel path ...")
        out["unfused"] = unfused_path(torch, tk, dev, w, n, fmt, sfmt, clamp, sets, args.steps // 4 or 1, stream,
                                      avg_launch_s)
    if not args.no_ceiling:
        log("[bench] streaming ceiling ...")
        ceil = stream_ceiling(torch, dev, n, w.hidden)
        out["roofline"]["measured_ceiling"] = ceil
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["read4_write1_GBs"], 4)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
