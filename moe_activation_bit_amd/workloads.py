"""Seeded synthetic workloads for the fused SwiGLU + top-k weight + FP8/FP4
cast and for the weighted top-k reduce of the experts' output rows.

This module only draws inputs (random streams, bf16 rounding of samples,
routing-weight normalisation, the position map of a dispatch layout); it
holds none of the activation, quantisation or reduce arithmetic.  The tests, the benchmark and the oracle's harness
all draw their inputs here, so both sides of every comparison see the same
bytes.

Shapes follow the MoE layout described in "【DeepSeek】TileKernels从入门到精通"
ch.2 (a packed ``[num_expanded_tokens, 2*hidden]`` bf16 tensor, gate on the
left half, up on the right half, one top-k weight per expanded row).

Every value is a pure function of (workload, seed, tensor name, element
index), so any row of a large tensor can be regenerated alone.
"""
from __future__ import annotations

import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SYNTH_LIB = os.path.join(_HERE, "libsynth.so")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distributions and cast options."""

    name: str
    rows: int                      # expanded rows (tokens x top-k); 0 = drawn per seed
    hidden: int
    sigma: float                   # std-dev of the bf16 activations
    fmt: str                       # "fp8" (E4M3) or "fp4" (E2M1)
    group_size: int                # 0 = one scale per row
    scale_fmt: str                 # "fp32" or "ue8m0"
    clamp_limit: Optional[float]   # None = no clamp
    weights: str                   # "uniform" | "renorm8" | "zero30"
    outlier_p: float = 0.0         # probability of replacing an element by +-outlier
    outlier_value: float = 0.0
    max_rows: int = 0              # for rows == 0: rows ~ U{1..max_rows}

    @property
    def code_bytes_per_row(self) -> int:
        return self.hidden if self.fmt == "fp8" else self.hidden // 2

    @property
    def groups_per_row(self) -> int:
        return 1 if self.group_size == 0 else self.hidden // self.group_size

    @property
    def scale_itemsize(self) -> int:
        return 4 if self.scale_fmt == "fp32" else 1

    def algorithmic_bytes(self, n: int) -> int:
        """Bytes the step must move at least once: x + topk_weight + codes + scales."""
        per_row = 4 * self.hidden + 4 + self.code_bytes_per_row + self.groups_per_row * self.scale_itemsize
        return n * per_row


WORKLOADS = {
    w.name: w
    for w in [
        # tiny per-token FP8 case, small enough for the oracle on every element
        Workload("fp8_per_token_n256_h1024", 256, 1024, 1.0, "fp8", 0, "fp32", None, "uniform"),
        # 4096 tokens x top-8, per-block FP8, power-of-two scales
        Workload("fp8_g128_ue8m0_n32768_h2048", 32768, 2048, 2.0, "fp8", 128, "ue8m0", None, "renorm8"),
        # 16384 tokens x top-8 prefill with 0.1% outliers at +-50 and clamp 10
        Workload("fp8_per_token_clamp10_n131072_h2048", 131072, 2048, 3.0, "fp8", 0, "fp32", 10.0,
                 "renorm8", outlier_p=0.001, outlier_value=50.0),
        # FP4 E2M1 per-block with power-of-two scales
        Workload("fp4_g32_ue8m0_n65536_h4096", 65536, 4096, 1.0, "fp4", 32, "ue8m0", None, "uniform"),
        # ragged decode batch: rows drawn per seed in [1, 1000], 30% zero weights
        Workload("fp8_g128_fp32_ragged_h7168", 0, 7168, 1.0, "fp8", 128, "fp32", None, "zero30",
                 max_rows=1000),
    ]
}

# The benchmark's headline workload: the largest configuration (16384 tokens x
# top-8 prefill, per-token FP8 with clamp 10: 1.34 GB moved per launch).
HEADLINE = "fp8_per_token_clamp10_n131072_h2048"

# Per-token rows longer than the workloads above use, 512 MiB of x each: one
# wave of 16 streamed 512-column steps per row; two waves of 16; four waves of
# 9 (a 12-step template).  Timed by `bench.py --workload NAME`, never by
# default.
LONG_ROW_WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp8_per_token_n16384_h8192", 16384, 8192, 3.0, "fp8", 0, "fp32", None, "uniform"),
        Workload("fp8_per_token_n8192_h16384", 8192, 16384, 3.0, "fp8", 0, "fp32", None, "uniform"),
        Workload("fp8_per_token_n7281_h18432", 7281, 18432, 3.0, "fp8", 0, "fp32", None, "uniform"),
    ]
}


def workload(name: str) -> Workload:
    """A fused-step workload by name, from either table."""
    return WORKLOADS[name] if name in WORKLOADS else LONG_ROW_WORKLOADS[name]


_lib = None


def _synth():
    global _lib
    if _lib is None:
        if not os.path.exists(SYNTH_LIB):
            raise RuntimeError(f"{SYNTH_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(SYNTH_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_char_p]
        lib.synth_u64.restype = ctypes.c_uint64
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_int64]
        lib.synth_uniform.restype = None
        lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_double, ctypes.c_void_p]
        lib.synth_outliers_bf16.restype = None
        lib.synth_outliers_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                            ctypes.c_void_p]
        _lib = lib
    return _lib


def stream_key(workload: str, seed: int, tensor: str) -> int:
    return _synth().synth_key(f"{workload}/{seed}/{tensor}".encode())


def uniform(key: int, first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    if count:
        _synth().synth_uniform(key, first, count, out.ctypes.data)
    return out


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def num_rows(w: Workload, seed: int) -> int:
    if w.rows:
        return w.rows
    u = uniform(stream_key(w.name, seed, "rows"), 0, 1)[0]
    return 1 + int(math.floor(u * w.max_rows))


def make_x(w: Workload, seed: int, rows: Optional[Sequence[int]] = None,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits of x, shape [len(rows), 2*hidden] (all rows when rows is None)."""
    lib = _synth()
    n = num_rows(w, seed)
    width = 2 * w.hidden
    if rows is None:
        row_list = None
        count_rows = n
    else:
        row_list = [int(r) for r in rows]
        count_rows = len(row_list)
    x = out if out is not None else np.empty((count_rows, width), dtype=np.uint16)
    assert x.shape == (count_rows, width) and x.dtype == np.uint16 and x.flags.c_contiguous
    k_norm = stream_key(w.name, seed, "x")
    k_p = stream_key(w.name, seed, "outlier_p")
    k_s = stream_key(w.name, seed, "outlier_sign")
    base = x.ctypes.data

    def fill(span):
        lo, hi = span  # local row range
        for i in range(lo, hi):
            r = i if row_list is None else row_list[i]
            ptr = base + i * width * 2
            first = r * width
            lib.synth_normal_bf16(k_norm, first, width, w.sigma, ptr)
            if w.outlier_p > 0:
                lib.synth_outliers_bf16(k_p, k_s, first, width, w.outlier_p, w.outlier_value, ptr)

    if count_rows:
        nt = min(_threads(), count_rows)
        step = (count_rows + nt - 1) // nt
        spans = [(i, min(count_rows, i + step)) for i in range(0, count_rows, step)]
        if len(spans) == 1:
            fill(spans[0])
        else:
            with ThreadPoolExecutor(len(spans)) as ex:
                list(ex.map(fill, spans))
    return x


def make_w(w: Workload, seed: int) -> np.ndarray:
    """fp32 top-k routing weights, shape [rows]."""
    n = num_rows(w, seed)
    u = uniform(stream_key(w.name, seed, "w"), 0, n)
    if w.weights == "uniform":
        out = u
    elif w.weights == "renorm8":
        # each token's 8 expanded rows are consecutive; its weights sum to 1
        out = np.empty(n, dtype=np.float64)
        for t0 in range(0, n, 8):
            grp = u[t0:t0 + 8]
            out[t0:t0 + 8] = grp / grp.sum()
    elif w.weights == "zero30":
        z = uniform(stream_key(w.name, seed, "w_zero"), 0, n)
        out = np.where(z < 0.3, 0.0, u)
    else:
        raise ValueError(w.weights)
    return out.astype(np.float32)


# ---------------------------------------------------------------------------
# Weighted top-k reduce of the experts' output rows
# ("【DeepSeek】TileKernels从入门到精通" ch.3 "结算中心的“减法工程”" and
# "动态寻址": the rows are found through a token/top-k -> position map).
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class ReduceWorkload:
    """One synthetic reduce workload.  The expanded rows are laid out as an MoE
    dispatch leaves them: grouped by expert, tokens in order within an expert,
    so a token's k rows lie far apart."""

    name: str
    tokens: int
    k: int
    experts: int
    hidden: int
    sigma: float                  # std-dev of the bf16 expert outputs
    drop_p: float                 # probability that a (token, slot) was dropped
    row_scale: bool               # a per-row dequantisation factor is given
    global_scale: float
    out_bf16: bool
    skew: float = 1.0             # expert popularity ~ (rank+1)^-skew

    def out_bytes_per_token(self) -> int:
        return self.hidden * (2 if self.out_bf16 else 4)

    def algorithmic_bytes(self, pos: np.ndarray) -> int:
        """Bytes the step must move at least once: the present rows (and their
        scale), the position map and weights, and the output."""
        present = int(np.count_nonzero(pos >= 0))
        per_present = 2 * self.hidden + (4 if self.row_scale else 0)
        return present * per_present + pos.size * 8 + self.tokens * self.out_bytes_per_token()


REDUCE_WORKLOADS = {
    r.name: r
    for r in [
        # small case for the oracle on every element: 64 tokens x top-8 of 256
        # experts, hidden 7168, 5% dropped slots
        ReduceWorkload("reduce_t64_k8_h7168_drop5", 64, 8, 256, 7168, 1.0, 0.05, True, 2.5, True),
        # 4096 tokens x top-8 of 256 experts at hidden 7168: the down-projection
        # outputs of the 32768 expanded rows of the headline activation step
        ReduceWorkload("reduce_t4096_k8_h7168", 4096, 8, 256, 7168, 1.0, 0.0, True, 2.5, True),
    ]
}
REDUCE_HEADLINE = "reduce_t4096_k8_h7168"


def make_routing(r: ReduceWorkload, seed: int):
    """(pos int32 [tokens, k], w fp32 [tokens, k], row_scale fp32 [n_rows] or
    None, n_rows).  Each token picks k distinct experts (popularity skewed by
    a power law); the present (token, slot) pairs get rows expert-major,
    tokens in order within an expert; dropped pairs get -1.  w is each
    token's uniform draws normalised to sum 1 (zero-weight dropped slots
    keep their draw)."""
    T, k, E = r.tokens, r.k, r.experts
    pop = (np.arange(E, dtype=np.float64) + 1.0) ** -r.skew
    perm = np.argsort(uniform(stream_key(r.name, seed, "expert_perm"), 0, E), kind="stable")
    pop = pop[np.argsort(perm, kind="stable")]  # popularity not tied to the expert index
    # k distinct experts per token: the k largest of u^(1/pop) (weighted draw
    # without replacement)
    u = uniform(stream_key(r.name, seed, "expert_pick"), 0, T * E).reshape(T, E)
    keys = np.log(np.maximum(u, 1e-300)) / pop
    experts = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int64)
    drop = uniform(stream_key(r.name, seed, "drop"), 0, T * k).reshape(T, k) < r.drop_p
    t_idx = np.repeat(np.arange(T, dtype=np.int64), k).reshape(T, k)
    present = ~drop
    e_p, t_p = experts[present], t_idx[present]
    order = np.lexsort((t_p, e_p))  # expert-major, then token
    rows = np.empty(order.size, dtype=np.int64)
    rows[order] = np.arange(order.size, dtype=np.int64)
    pos = np.full((T, k), -1, dtype=np.int32)
    pos[present] = rows.astype(np.int32)
    n_rows = int(order.size)
    wu = uniform(stream_key(r.name, seed, "w"), 0, T * k).reshape(T, k)
    w = (wu / wu.sum(axis=1, keepdims=True)).astype(np.float32)
    rs = None
    if r.row_scale:
        rs = (0.5 + 1.5 * uniform(stream_key(r.name, seed, "row_scale"), 0, n_rows)).astype(np.float32)
    return pos, w, rs, n_rows


def make_expert_rows(r: ReduceWorkload, seed: int, n_rows: int, rows: Optional[Sequence[int]] = None,
                     out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits of the experts' output rows, shape [n_rows, hidden] (or the
    listed rows only)."""
    lib = _synth()
    hidden = r.hidden
    row_list = list(range(n_rows)) if rows is None else [int(i) for i in rows]
    x = out if out is not None else np.empty((len(row_list), hidden), dtype=np.uint16)
    assert x.shape == (len(row_list), hidden) and x.dtype == np.uint16 and x.flags.c_contiguous
    key = stream_key(r.name, seed, "expert_rows")
    base = x.ctypes.data

    def fill(span):
        for i in range(*span):
            lib.synth_normal_bf16(key, row_list[i] * hidden, hidden, r.sigma, base + i * hidden * 2)

    count = len(row_list)
    if count:
        nt = min(_threads(), count)
        step = (count + nt - 1) // nt
        spans = [(i, min(count, i + step)) for i in range(0, count, step)]
        with ThreadPoolExecutor(len(spans)) as ex:
            list(ex.map(fill, spans))
    return x
