"""The oracle: a plain CPU statement of the fused SwiGLU + top-k weight +
FP8/FP4 cast, the stand-alone cast, the top-k gating and the weighted top-k
reduce (see oracle.c for the sources it follows and every reading it takes).  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
benchmark's CPU-baseline leg may use it; the GPU library never does.

numpy in, numpy out.  x is the bf16 bit pattern as uint16 [n, 2*hidden].
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the wrapper at another build of oracle.c (the mutation
# test loads copies with planted mistakes this way).
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")

FP8 = 8
FP4 = 4
SCALE_FP32 = 0
SCALE_UE8M0 = 1
FMT_MAX = {FP8: 448.0, FP4: 6.0}

_lib = None


def build_command(out: str = os.path.join(_HERE, "liboracle.so"), source: str = SOURCE) -> list:
    return ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-o", out, source,
            "-lquadmath", "-lm"]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        c = ctypes
        lib.oracle_sigmoid.restype = c.c_float
        lib.oracle_sigmoid.argtypes = [c.c_float]
        lib.oracle_e4m3.restype = c.c_uint8
        lib.oracle_e4m3.argtypes = [c.c_float]
        lib.oracle_e2m1.restype = c.c_uint8
        lib.oracle_e2m1.argtypes = [c.c_float]
        lib.oracle_ue8m0_exponent.restype = c.c_int
        lib.oracle_ue8m0_exponent.argtypes = [c.c_float, c.c_float]
        lib.oracle_encode.restype = c.c_int
        lib.oracle_encode.argtypes = [c.c_int, c.c_void_p, c.c_int64, c.c_void_p]
        lib.oracle_swiglu_forward.restype = c.c_int
        lib.oracle_swiglu_forward.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_float,
                                              c.c_void_p, c.c_void_p]
        lib.oracle_cast.restype = c.c_int
        lib.oracle_cast.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_int, c.c_int,
                                    c.c_void_p, c.c_void_p]
        lib.oracle_cast_bf16.restype = c.c_int
        lib.oracle_cast_bf16.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_int, c.c_int,
                                         c.c_void_p, c.c_void_p]
        lib.oracle_topk_gate.restype = c.c_int
        lib.oracle_topk_gate.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_int64, c.c_int64,
                                         c.c_int, c.c_void_p, c.c_void_p]
        lib.oracle_moe_reduce.restype = c.c_int
        lib.oracle_topk_to_pos.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p]
        lib.oracle_topk_to_pos.restype = c.c_int
        lib.oracle_moe_reduce.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_float, c.c_int64,
                                          c.c_int64, c.c_int64, c.c_int64, c.c_int, c.c_void_p]
        lib.oracle_swiglu_cast.restype = c.c_int
        lib.oracle_swiglu_cast.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int64,
                                           c.c_float, c.c_int, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p]
        _lib = lib
    return _lib


def sigmoid(g: float) -> float:
    return float(np.float32(_load().oracle_sigmoid(float(g))))


def e4m3(q: float) -> int:
    return int(_load().oracle_e4m3(float(q)))


def e2m1(q: float) -> int:
    return int(_load().oracle_e2m1(float(q)))


def encode(q: np.ndarray, fmt: int) -> np.ndarray:
    """One code byte per fp32 value (E4M3 for fmt 8, E2M1 for fmt 4)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape, dtype=np.uint8)
    if _load().oracle_encode(fmt, q.ctypes.data, q.size, out.ctypes.data):
        raise ValueError("oracle_encode failed")
    return out


def ue8m0_exponent(amax: float, fmt: int) -> int:
    return int(_load().oracle_ue8m0_exponent(float(amax), FMT_MAX[fmt]))


def _clamp_arg(clamp_limit: Optional[float]) -> float:
    return math.inf if clamp_limit is None else float(clamp_limit)


def _x(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16 and x.ndim == 2 and x.shape[1] % 2 == 0
    return x


def _w(w: Optional[np.ndarray], n: int) -> Optional[np.ndarray]:
    if w is None:
        return None
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape == (n,)
    return w


def swiglu_forward(x: np.ndarray, w: Optional[np.ndarray],
                   clamp_limit: Optional[float] = None) -> Tuple[np.ndarray, int]:
    """First stage of the unfused reference: fp32 y [n, hidden] and the clamp count."""
    x = _x(x)
    n, hidden = x.shape[0], x.shape[1] // 2
    w = _w(w, n)
    y = np.empty((n, hidden), dtype=np.float32)
    cnt = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_swiglu_forward(x.ctypes.data, None if w is None else w.ctypes.data, n, hidden,
                                       _clamp_arg(clamp_limit), y.ctypes.data, cnt.ctypes.data)
    if rc:
        raise ValueError(f"oracle_swiglu_forward failed ({rc})")
    return y, int(cnt[0])


def _out(n: int, hidden: int, group_size: int, fmt: int, scale_fmt: int):
    groups = 1 if group_size == 0 else hidden // group_size
    codes = np.empty((n, hidden if fmt == FP8 else hidden // 2), dtype=np.uint8)
    scales = np.empty((n, groups), dtype=np.float32 if scale_fmt == SCALE_FP32 else np.uint8)
    return codes, scales


def cast(y: np.ndarray, group_size: int, fmt: int, scale_fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    """Second stage of the unfused reference: codes and scales from fp32 rows."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    n, hidden = y.shape
    codes, scales = _out(n, hidden, group_size, fmt, scale_fmt)
    rc = _load().oracle_cast(y.ctypes.data, n, hidden, group_size, fmt, scale_fmt, codes.ctypes.data,
                             scales.ctypes.data)
    if rc:
        raise ValueError(f"oracle_cast failed ({rc})")
    return codes, scales


def cast_bf16(x: np.ndarray, group_size: int, fmt: int, scale_fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    """The stand-alone cast of bf16 rows (uint16 bit patterns [n, hidden])."""
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16 and x.ndim == 2
    n, hidden = x.shape
    codes, scales = _out(n, hidden, group_size, fmt, scale_fmt)
    rc = _load().oracle_cast_bf16(x.ctypes.data, n, hidden, group_size, fmt, scale_fmt, codes.ctypes.data,
                                  scales.ctypes.data)
    if rc:
        raise ValueError(f"oracle_cast_bf16 failed ({rc})")
    return codes, scales


def scale_layout(scales: np.ndarray, layout: str, fill: int = 0) -> np.ndarray:
    """Row-major scales [n, G] (fp32 or UE8M0 bytes) re-laid as the scale
    tensor of the given layout, returned as raw bytes; positions the layout
    leaves unwritten hold `fill`.  Data movement only:
      "fp32_colmajor"  fp32  [G][ld], ld = n rounded up to 4, (r, k) at k*ld + r
      "ue8m0_colmajor" uint8 [G][ld], ld = n rounded up to 16
      "ue8m0_packed"   uint32 [ceil(G/4)][ld], ld = n rounded up to 4; word (j, r)
                       holds the bytes of groups 4j..4j+3 of row r, group 4j lowest
    """
    n, G = scales.shape
    if layout == "fp32_colmajor":
        ld = (n + 3) // 4 * 4
        out = np.full((G, ld, 4), fill, dtype=np.uint8)
        for k in range(G):
            for r in range(n):
                out[k, r] = np.frombuffer(np.float32(scales[r, k]).tobytes(), dtype=np.uint8)
        return out.reshape(-1)
    if layout == "ue8m0_colmajor":
        ld = (n + 15) // 16 * 16
        out = np.full((G, ld), fill, dtype=np.uint8)
        for k in range(G):
            for r in range(n):
                out[k, r] = scales[r, k]
        return out.reshape(-1)
    if layout == "ue8m0_packed":
        ld = (n + 3) // 4 * 4
        out = np.full(((G + 3) // 4, ld, 4), fill, dtype=np.uint8)
        for k in range(G):
            for r in range(n):
                out[k // 4, r, k % 4] = scales[r, k]
        return out.reshape(-1)
    raise ValueError(layout)


def swiglu_cast(x: np.ndarray, w: Optional[np.ndarray], group_size: int, clamp_limit: Optional[float],
                fmt: int, scale_fmt: int) -> Tuple[np.ndarray, np.ndarray, int]:
    """The fused step, row by row: (codes, scales, clamped_count)."""
    x = _x(x)
    n, hidden = x.shape[0], x.shape[1] // 2
    w = _w(w, n)
    codes, scales = _out(n, hidden, group_size, fmt, scale_fmt)
    cnt = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_swiglu_cast(x.ctypes.data, None if w is None else w.ctypes.data, n, hidden,
                                    group_size, _clamp_arg(clamp_limit), fmt, scale_fmt,
                                    codes.ctypes.data, scales.ctypes.data, cnt.ctypes.data)
    if rc:
        raise ValueError(f"oracle_swiglu_cast failed ({rc})")
    return codes, scales, int(cnt[0])


def topk_gate(scores: np.ndarray, k: int, n_group: int = 1, topk_group: int = 1,
              normalise: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k expert selection per token (oracle.c: oracle_topk_gate):
    (indices int32 [tokens, k], weights fp32 [tokens, k]), best first."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    tokens, experts = scores.shape
    idx = np.empty((tokens, k), dtype=np.int32)
    w = np.empty((tokens, k), dtype=np.float32)
    rc = _load().oracle_topk_gate(scores.ctypes.data, tokens, experts, k, n_group, topk_group, int(normalise),
                                  idx.ctypes.data, w.ctypes.data)
    if rc:
        raise ValueError(f"oracle_topk_gate failed ({rc})")
    return idx, w


def moe_reduce(x: np.ndarray, pos: np.ndarray, w: np.ndarray, row_scale: Optional[np.ndarray] = None,
               global_scale: float = 1.0, out_bf16: bool = True) -> np.ndarray:
    """Weighted top-k reduce (oracle.c: oracle_moe_reduce).  x: bf16 bits uint16
    [n_rows, hidden]; pos: int32 [tokens, k] row per (token, slot), entries
    outside [0, n_rows) dropped; w: fp32 [tokens, k]; row_scale: fp32 [n_rows]
    or None.  Returns bf16 bits uint16 [tokens, hidden], or fp32."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n_rows, hidden = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    tokens, k = pos.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape == (tokens, k)
    rs = None
    if row_scale is not None:
        rs = np.ascontiguousarray(row_scale, dtype=np.float32)
        assert rs.shape == (n_rows,)
    out = np.empty((tokens, hidden), dtype=np.uint16 if out_bf16 else np.float32)
    rc = _load().oracle_moe_reduce(x.ctypes.data, None if rs is None else rs.ctypes.data, pos.ctypes.data,
                                   w.ctypes.data, float(global_scale), tokens, k, hidden, n_rows, int(out_bf16),
                                   out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_moe_reduce failed ({rc})")
    return out


def topk_to_pos(idx: np.ndarray, experts: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token/top-k -> expert-row map (oracle.c: oracle_topk_to_pos):
    (pos int32 [tokens, k], -1 for absent slots; offsets int32 [experts + 1])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    tokens, k = idx.shape
    pos = np.empty((tokens, k), dtype=np.int32)
    off = np.empty((experts + 1,), dtype=np.int32)
    rc = _load().oracle_topk_to_pos(idx.ctypes.data, tokens, k, experts, pos.ctypes.data, off.ctypes.data)
    if rc:
        raise ValueError(f"oracle_topk_to_pos failed ({rc})")
    return pos, off
