"""Python binding of the MI355X fused SwiGLU + top-k weight + FP8/FP4 cast,
the stand-alone cast, the top-k gating and the weighted top-k reduce.

Argument marshalling only: every function here forwards to the C ABI in
``include/tk.h`` (library ``libtk.so`` built from ``csrc/*.hip``) under the
same name, through the small CPython extension ``_tkpy`` (``csrc/tk_py.c``,
a fraction of a microsecond per call where ctypes took a few).  All
arithmetic runs in the library's HIP kernels; there is no CPU fallback, and
calling a function whose library or extension is missing raises.

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed) or raw
device addresses as ints; ``None`` is a null pointer.  ``stream`` defaults to
torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import enum
import os
from typing import Any, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtk.so")

__all__ = [
    "TkStatus", "TK_SCALE_FP32", "TK_SCALE_UE8M0", "TK_SCALE_FP32_COLMAJOR", "TK_SCALE_UE8M0_COLMAJOR",
    "TK_SCALE_UE8M0_PACKED", "TK_DTYPE_BF16", "TK_DTYPE_FP32", "LIB_PATH", "load_library", "load_extension",
    "tk_init", "tk_swiglu_cast_fp8", "tk_swiglu_cast_fp4", "tk_swiglu_forward", "tk_cast_fp8", "tk_cast_fp4",
    "tk_topk_gate", "tk_moe_reduce", "tk_status_str",
]

TK_SCALE_FP32 = 0
TK_SCALE_UE8M0 = 1
TK_SCALE_FP32_COLMAJOR = 2
TK_SCALE_UE8M0_COLMAJOR = 3
TK_SCALE_UE8M0_PACKED = 4
TK_DTYPE_BF16 = 0
TK_DTYPE_FP32 = 1


class TkStatus(enum.IntEnum):
    TK_OK = 0
    TK_ERR_INVALID_ARG = 1
    TK_ERR_UNSUPPORTED = 2
    TK_ERR_HIP = 3


_lib: Optional[ctypes.CDLL] = None

# the exported symbols and their C signatures, as declared in include/tk.h
_CAST_ARGS = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
              ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
              ctypes.c_void_p]
SIGNATURES = {
    "tk_init": (ctypes.c_int, [ctypes.c_int]),
    "tk_swiglu_cast_fp8": (ctypes.c_int, _CAST_ARGS),
    "tk_swiglu_cast_fp4": (ctypes.c_int, _CAST_ARGS),
    "tk_swiglu_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_cast_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_cast_fp4": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_topk_gate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_moe_reduce": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_float, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_topk_to_pos": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tk_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}


def load_library() -> ctypes.CDLL:
    """Load libtk.so (fails loudly when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


EXT_NAME = "_tkpy"  # the CPython extension that marshals arguments to libtk.so (csrc/tk_py.c)
_ext = None
_STATUS = tuple(TkStatus(i) for i in range(len(TkStatus)))


def _current_stream() -> int:
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def load_extension():
    """Import the argument-marshalling extension (fails loudly when it has not
    been built); its default stream is torch's current stream."""
    global _ext
    if _ext is None:
        load_library()
        import importlib
        try:
            mod = importlib.import_module(f"{__name__}.{EXT_NAME}")
        except ImportError as e:
            raise RuntimeError(f"{EXT_NAME} is missing: build the package first (__graft_entry__.build())") from e
        mod._set_stream_getter(_current_stream)
        _ext = mod
    return _ext


# Pointer arguments: a torch tensor (its data_ptr()), an int address or None.
# stream: None (torch's current stream), an int handle or a torch stream.


def tk_init(device: int) -> TkStatus:
    return _STATUS[(_ext or load_extension()).tk_init(int(device))]


def tk_swiglu_cast_fp8(x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales,
                       clamped_count=None, stream=None) -> TkStatus:
    """See tk_swiglu_cast_fp8 in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_swiglu_cast_fp8(
        x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales, clamped_count, stream)]


def tk_swiglu_cast_fp4(x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales,
                       clamped_count=None, stream=None) -> TkStatus:
    """See tk_swiglu_cast_fp4 in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_swiglu_cast_fp4(
        x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales, clamped_count, stream)]


def tk_swiglu_forward(x, topk_weight, n, hidden, clamp_limit, y, clamped_count=None,
                      stream=None) -> TkStatus:
    """See tk_swiglu_forward in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_swiglu_forward(x, topk_weight, n, hidden, clamp_limit, y,
                                                                  clamped_count, stream)]


def tk_cast_fp8(x, in_dtype, n, hidden, group_size, scale_fmt, codes, scales, stream=None) -> TkStatus:
    """See tk_cast_fp8 in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_cast_fp8(x, in_dtype, n, hidden, group_size, scale_fmt, codes,
                                                            scales, stream)]


def tk_cast_fp4(x, in_dtype, n, hidden, group_size, scale_fmt, codes, scales, stream=None) -> TkStatus:
    """See tk_cast_fp4 in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_cast_fp4(x, in_dtype, n, hidden, group_size, scale_fmt, codes,
                                                            scales, stream)]


def tk_topk_gate(scores, tokens, experts, k, n_group, topk_group, normalise, topk_idx, topk_weight,
                 stream=None) -> TkStatus:
    """See tk_topk_gate in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_topk_gate(scores, tokens, experts, k, n_group, topk_group,
                                                             normalise, topk_idx, topk_weight, stream)]


def tk_moe_reduce(x, row_scale, pos, topk_weight, global_scale, tokens, k, hidden, n_rows, out_dtype, out,
                  stream=None) -> TkStatus:
    """See tk_moe_reduce in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_moe_reduce(x, row_scale, pos, topk_weight, global_scale, tokens,
                                                              k, hidden, n_rows, out_dtype, out, stream)]


def tk_topk_to_pos(topk_idx, tokens, k, experts, pos, expert_offsets, stream=None) -> TkStatus:
    """See tk_topk_to_pos in include/tk.h."""
    return _STATUS[(_ext or load_extension()).tk_topk_to_pos(topk_idx, tokens, k, experts, pos, expert_offsets,
                                                               stream)]


def tk_status_str(status: int) -> str:
    return (_ext or load_extension()).tk_status_str(int(status))
