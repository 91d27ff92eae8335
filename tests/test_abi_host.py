"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/tk.h declares, and rejects bad arguments before making
any HIP call (fake, never-dereferenced device addresses are used)."""
import math
import os
import re

import pytest

import moe_activation_bit_amd as tk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tk.h")

OK, INVALID, UNSUPPORTED = tk.TkStatus.TK_OK, tk.TkStatus.TK_ERR_INVALID_ARG, tk.TkStatus.TK_ERR_UNSUPPORTED
FP32, UE8M0 = tk.TK_SCALE_FP32, tk.TK_SCALE_UE8M0
INF = math.inf

# fake device addresses: aligned, far apart, never dereferenced.  Every call
# given them is rejected before any HIP call or has no rows to process, so no
# kernel is ever launched on them (a supported shape is checked with n = 0).
X, W, C, S, K = 0x7000_0000_0000, 0x7100_0000_0000, 0x7200_0000_0000, 0x7300_0000_0000, 0x7400_0000_0000


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:tk_status|const char\s*\*)\s*(tk_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(["tk_init", "tk_status_str", "tk_swiglu_cast_fp4", "tk_swiglu_cast_fp8",
                                         "tk_swiglu_forward", "tk_cast_fp8", "tk_cast_fp4", "tk_topk_gate",
                                         "tk_moe_reduce", "tk_topk_to_pos"])


def test_library_exports_every_declared_symbol():
    lib = tk.load_library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in tk.SIGNATURES, name
        assert callable(getattr(tk, name)), name  # binding of the same name


def test_status_strings():
    for st in tk.TkStatus:
        assert tk.tk_status_str(st) == st.name
    assert tk.tk_status_str(99) == "TK_UNKNOWN_STATUS"


def cast8(**kw):
    a = dict(x=X, topk_weight=W, n=4, hidden=1024, group_size=0, clamp_limit=INF, scale_fmt=FP32, codes=C,
             scales=S, clamped_count=None, stream=0)
    a.update(kw)
    return tk.tk_swiglu_cast_fp8(**a)


def cast4(**kw):
    a = dict(x=X, topk_weight=W, n=4, hidden=1024, group_size=32, clamp_limit=INF, scale_fmt=UE8M0, codes=C,
             scales=S, clamped_count=None, stream=0)
    a.update(kw)
    return tk.tk_swiglu_cast_fp4(**a)


@pytest.mark.parametrize("kw", [
    dict(n=-1), dict(n=2 ** 31), dict(hidden=0), dict(hidden=-8), dict(hidden=12), dict(group_size=-8),
    dict(group_size=12), dict(group_size=48), dict(clamp_limit=float("nan")), dict(clamp_limit=0.0),
    dict(clamp_limit=-1.0), dict(clamp_limit=-INF), dict(scale_fmt=7), dict(scale_fmt=-1), dict(x=None),
    dict(codes=None), dict(scales=S + 4, scale_fmt=tk.TK_SCALE_FP32_COLMAJOR),
    dict(scales=S + 8, scale_fmt=tk.TK_SCALE_UE8M0_COLMAJOR), dict(scales=S + 4, scale_fmt=tk.TK_SCALE_UE8M0_PACKED),
    dict(scales=None), dict(x=X + 8), dict(codes=C + 4), dict(topk_weight=W + 2), dict(clamped_count=K + 4),
    dict(codes=X), dict(scales=X + 64), dict(codes=W), dict(scales=C + 16), dict(clamped_count=S),
], ids=str)
def test_fp8_invalid_arguments(kw):
    assert cast8(**kw) == INVALID


@pytest.mark.parametrize("kw", [
    dict(hidden=1028), dict(codes=C + 2), dict(group_size=24), dict(scales=S + 1, scale_fmt=FP32),
], ids=str)
def test_fp4_invalid_arguments(kw):
    assert cast4(**kw) == INVALID


def test_ue8m0_scales_need_no_alignment_and_n0_is_a_noop():
    # n == 0 returns before any HIP call, with or without pointers
    assert cast8(n=0) == OK
    assert cast8(n=0, x=None, codes=None, scales=None) == OK
    assert cast4(n=0, scales=S + 1) == OK


@pytest.mark.parametrize("kw", [
    dict(hidden=48, group_size=24),        # 3 lane slots per group: segmented units
    dict(hidden=1536, group_size=768),     # 96 slots: segmented
    dict(hidden=7168, group_size=896),     # 112 slots: segmented, a group straddles steps
    dict(hidden=9600, group_size=4800),    # 600 slots: segmented, 16 steps per unit
    dict(hidden=17600, group_size=8800),   # 1100 slots, not whole steps: two-pass
    dict(hidden=32776, group_size=0),      # per-token group longer than 32768 columns: two-pass
    dict(hidden=40960, group_size=40960),
    dict(hidden=17408, group_size=8704),   # two groups of 17 steps (odd): two-pass
    dict(hidden=34816, group_size=17408),  # two groups of 34 steps (not a multiple of 4): two-pass
    dict(hidden=8200, group_size=0),       # 17 steps: two waves
    dict(hidden=32768, group_size=0),      # 64 steps: four waves
    dict(hidden=16384, group_size=16384),
    dict(hidden=17408, group_size=17408),  # one group of 34 steps: four waves, the last short
    dict(hidden=36864, group_size=18432),  # two groups of 36 steps
    dict(hidden=32768, group_size=16384),  # two groups of 32 steps
], ids=str)
def test_every_valid_group_is_planned(kw):
    # every group width that is a multiple of 8 dividing hidden has a kernel;
    # with n == 0 the call returns after planning, before any HIP call
    assert cast8(n=0, **kw) == OK
    assert cast4(n=0, **kw) == OK
    assert cast_only(tk.tk_cast_fp8, n=0, **kw) == OK
    assert cast_only(tk.tk_cast_fp4, n=0, **kw) == OK


@pytest.mark.parametrize("kw", [dict(n=-1), dict(hidden=4), dict(y=None), dict(y=X + 4), dict(y=X),
                                dict(clamp_limit=float("nan"))], ids=str)
def test_swiglu_forward_invalid_arguments(kw):
    a = dict(x=X, topk_weight=W, n=4, hidden=1024, clamp_limit=INF, y=C, clamped_count=None, stream=0)
    a.update(kw)
    assert tk.tk_swiglu_forward(**a) == INVALID


def test_init_rejects_bad_device():
    # tk_init validates the index against the device count (0 here: no GPU)
    assert tk.tk_init(-1) in (INVALID, tk.TkStatus.TK_ERR_HIP)


def cast_only(fn, **kw):
    a = dict(x=X, in_dtype=tk.TK_DTYPE_BF16, n=4, hidden=1024, group_size=128, scale_fmt=UE8M0, codes=C, scales=S,
             stream=0)
    a.update(kw)
    return fn(**a)


@pytest.mark.parametrize("kw", [
    dict(n=-1), dict(hidden=12), dict(group_size=12), dict(in_dtype=2), dict(in_dtype=-1), dict(scale_fmt=5),
    dict(scales=S + 4, scale_fmt=tk.TK_SCALE_UE8M0_PACKED),
    dict(x=None), dict(codes=None), dict(scales=None), dict(x=X + 8), dict(codes=C + 2),
    dict(scales=S + 2, scale_fmt=FP32), dict(codes=X), dict(scales=X + 100), dict(codes=S),
], ids=str)
def test_cast_invalid_arguments(kw):
    # every case is invalid for both formats, so no call can reach a launch
    assert cast_only(tk.tk_cast_fp8, **kw) == INVALID
    assert cast_only(tk.tk_cast_fp4, **kw) == INVALID


def test_cast_empty():
    assert cast_only(tk.tk_cast_fp8, n=0, hidden=48, group_size=24) == OK
    assert cast_only(tk.tk_cast_fp8, n=0, hidden=32776, group_size=0) == OK
    assert cast_only(tk.tk_cast_fp8, n=0, hidden=8200, group_size=0) == OK
    assert cast_only(tk.tk_cast_fp8, n=0) == OK
    assert cast_only(tk.tk_cast_fp4, n=0, x=None, codes=None, scales=None) == OK


def topk(**kw):
    a = dict(scores=X, tokens=4, experts=256, k=8, n_group=8, topk_group=4, normalise=0, topk_idx=C, topk_weight=S,
             stream=0)
    a.update(kw)
    return tk.tk_topk_gate(**a)


@pytest.mark.parametrize("kw", [
    dict(tokens=-1), dict(experts=0), dict(k=0), dict(n_group=0), dict(topk_group=0), dict(n_group=3),
    dict(topk_group=9), dict(k=129), dict(experts=8, n_group=8, topk_group=1, k=1), dict(scores=None),
    dict(topk_idx=None), dict(topk_weight=None), dict(scores=X + 2), dict(topk_idx=X), dict(topk_weight=C + 8),
], ids=str)
def test_topk_invalid_arguments(kw):
    assert topk(**kw) == INVALID


def test_topk_unsupported_and_empty():
    assert topk(experts=576, n_group=8) == UNSUPPORTED     # more than 8 experts per lane
    assert topk(tokens=0, experts=512, n_group=8) == OK     # 8 per lane, groups of 8 lanes
    assert topk(tokens=0, experts=384, n_group=1, topk_group=1) == OK
    assert topk(experts=256, n_group=1, topk_group=1, k=65) == UNSUPPORTED
    assert topk(experts=72, n_group=8, topk_group=2, k=5) == UNSUPPORTED  # 9 experts per group: no layout
    assert topk(tokens=0, experts=72, n_group=3, topk_group=2, k=5) == OK  # 3 per lane, 8 lanes per group
    assert topk(tokens=0, experts=160, n_group=8, topk_group=3, k=6) == OK  # 5 per lane, 4 lanes per group
    assert topk(tokens=0, experts=100, n_group=5, topk_group=2, k=5) == OK  # 5 per lane (above the minimum 4)
    assert topk(tokens=0) == OK


def reduce(**kw):
    a = dict(x=X, row_scale=W, pos=C, topk_weight=S, global_scale=2.5, tokens=4, k=8, hidden=7168, n_rows=32,
             out_dtype=tk.TK_DTYPE_BF16, out=K, stream=0)
    a.update(kw)
    return tk.tk_moe_reduce(**a)


@pytest.mark.parametrize("kw", [
    dict(tokens=-1), dict(tokens=2 ** 31), dict(k=0), dict(k=-3), dict(hidden=0), dict(hidden=12), dict(hidden=-8),
    dict(n_rows=-1), dict(n_rows=2 ** 31), dict(out_dtype=2), dict(out_dtype=-1), dict(global_scale=float("nan")),
    dict(global_scale=INF), dict(pos=None), dict(topk_weight=None), dict(out=None), dict(x=None),
    dict(x=X + 8), dict(out=K + 8), dict(pos=C + 2), dict(topk_weight=S + 1), dict(row_scale=W + 2),
    dict(out=X + 64), dict(out=C), dict(out=S + 4), dict(out=W), dict(k=40, out=X),
], ids=str)
def test_moe_reduce_invalid_arguments(kw):
    assert reduce(**kw) == INVALID


def test_moe_reduce_unsupported_and_empty():
    assert reduce(k=65) == UNSUPPORTED
    assert reduce(k=1000) == UNSUPPORTED
    assert reduce(tokens=0) == OK
    assert reduce(tokens=0, x=None, pos=None, topk_weight=None, out=None) == OK
    # n_rows == 0 lets x be NULL (nothing can be read); with no tokens nothing launches
    assert reduce(tokens=0, n_rows=0, x=None) == OK


def to_pos(**kw):
    a = dict(topk_idx=X, tokens=4, k=8, experts=256, pos=C, expert_offsets=S, stream=0)
    a.update(kw)
    return tk.tk_topk_to_pos(**a)


@pytest.mark.parametrize("kw", [
    dict(tokens=-1), dict(tokens=2 ** 31), dict(k=0), dict(k=-1), dict(experts=0), dict(experts=-4),
    dict(tokens=2 ** 28), dict(topk_idx=None), dict(pos=None), dict(expert_offsets=None), dict(topk_idx=X + 2),
    dict(pos=C + 1), dict(expert_offsets=S + 3), dict(pos=X + 64), dict(expert_offsets=C + 4), dict(expert_offsets=X),
], ids=str)
def test_topk_to_pos_invalid_arguments(kw):
    # (an empty call is not made here: it launches a kernel to zero the offsets)
    assert to_pos(**kw) == INVALID


def test_topk_to_pos_unsupported():
    assert to_pos(k=65) == UNSUPPORTED
    assert to_pos(experts=513) == UNSUPPORTED


class _FakeTensor:
    """Stands in for a torch tensor: the binding takes its data_ptr()."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_extension_marshals_like_the_c_abi():
    # the binding goes through the _tkpy extension; its conversions must reach
    # the C ABI unchanged: objects with data_ptr(), ints and None for pointers,
    # numpy integers and floats for sizes, and the status comes back as TkStatus
    import numpy as np

    ext = tk.load_extension()
    assert os.path.dirname(ext.__file__) == os.path.dirname(tk.LIB_PATH)
    rc = tk.tk_swiglu_cast_fp8(_FakeTensor(X), _FakeTensor(W), np.int64(0), np.int32(1024), 0, np.float32(INF),
                               FP32, _FakeTensor(C), S, None, 0)
    assert rc is OK
    # a misaligned address passed as an object is rejected by the library itself
    assert tk.tk_swiglu_cast_fp8(_FakeTensor(X + 4), W, 4, 1024, 0, INF, FP32, C, S, None, 0) is INVALID
    assert tk.tk_cast_fp8(X, tk.TK_DTYPE_BF16, 0, 1024, 128, UE8M0, C, S, 0) is OK
    assert tk.tk_topk_gate(X, 0, 256, 8, 8, 4, True, C, S, 0) is OK
    assert tk.tk_moe_reduce(X, None, C, W, 1.0, 0, 8, 7168, 0, tk.TK_DTYPE_BF16, S, 0) is OK
    assert tk.tk_swiglu_forward(X, None, 0, 1024, INF, C, None, 0) is OK


@pytest.mark.parametrize("bad", [dict(x="not a pointer"), dict(n="4"), dict(clamp_limit="inf"), dict(scale_fmt=0.5),
                                 dict(stream="stream")], ids=str)
def test_extension_rejects_wrong_argument_types(bad):
    a = dict(x=X, topk_weight=W, n=4, hidden=1024, group_size=0, clamp_limit=INF, scale_fmt=FP32, codes=C,
             scales=S, clamped_count=None, stream=0)
    a.update(bad)
    with pytest.raises((TypeError, AttributeError)):
        tk.tk_swiglu_cast_fp8(**a)
