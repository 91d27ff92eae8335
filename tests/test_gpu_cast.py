"""GPU parity of the stand-alone cast (tk_cast_fp8 / tk_cast_fp4) and of the
unfused two-kernel path (tk_swiglu_forward then tk_cast) against the oracle
and against the fused kernel.  Bit-exact throughout."""
import math

import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
import oracle
from moe_activation_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAD = 256
OK = tk.TkStatus.TK_OK


def say(*a):
    print("[gpu-case]", *a, flush=True)


def run_cast(xd, in_dtype, n, hidden, group, fmt, sfmt):
    groups = 1 if group == 0 else hidden // group
    cols = hidden if fmt == 8 else hidden // 2
    sitem = 4 if sfmt == tk.TK_SCALE_FP32 else 1
    cbuf = torch.full((n * cols + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((n * groups * sitem + 2 * PAD,), 0x5A, dtype=torch.uint8, device=DEV)
    fn = tk.tk_cast_fp8 if fmt == 8 else tk.tk_cast_fp4
    rc = fn(xd, in_dtype, n, hidden, group, sfmt, cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD)
    assert rc == OK, tk.tk_status_str(rc)
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (c[:PAD] == 0xA5).all() and (c[len(c) - PAD:] == 0xA5).all(), "codes canary overwritten"
    assert (s[:PAD] == 0x5A).all() and (s[len(s) - PAD:] == 0x5A).all(), "scales canary overwritten"
    sb = s[PAD:len(s) - PAD]
    return c[PAD:len(c) - PAD].reshape(n, cols), (sb.view(np.float32) if sitem == 4 else sb).reshape(n, groups)


def same(got, want, what):
    gc, gs = got
    wc, ws = want
    if not np.array_equal(gc, wc):
        bad = np.argwhere(gc != wc)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first row {r} col {c}: {gc[r, c]:#x} vs {wc[r, c]:#x}")
    assert np.array_equal(gs.view(np.uint8), ws.view(np.uint8)), f"{what}: scales differ"


CASES = [  # (hidden, group, fmt, scale_fmt)
    (2048, 128, 8, 1), (2048, 0, 8, 0), (4096, 32, 4, 1), (7168, 128, 8, 0), (1000, 8, 4, 0), (1000, 0, 8, 1),
    (2048, 1024, 4, 1), (64, 32, 8, 0), (8192, 0, 4, 0), (6144, 0, 8, 1), (5000, 0, 4, 0),
    # groups that straddle lanes and steps (segmented units) and groups read twice (two-pass)
    (1944, 24, 8, 1), (1944, 24, 4, 0), (2040, 40, 4, 1), (2976, 96, 8, 0), (7168, 896, 8, 1), (7168, 896, 4, 0),
    (9600, 4800, 8, 0), (17600, 8800, 4, 1), (17408, 8704, 8, 1), (32776, 0, 8, 0), (40960, 0, 4, 1),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_cast_bf16_matches_oracle(case):
    hidden, group, fmt, sfmt = case
    say("cast bf16", case)
    base = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    rows = 77
    full = wl.make_x(base, 6, rows=range(rows))
    x = np.ascontiguousarray(np.tile(full, (1, (hidden + 4095) // 4096))[:, :hidden])
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    got = run_cast(xd, tk.TK_DTYPE_BF16, rows, hidden, group, fmt, sfmt)
    same(got, oracle.cast_bf16(x, group, fmt, sfmt), f"bf16 {case}")


@pytest.mark.parametrize("case", CASES, ids=str)
def test_cast_fp32_matches_oracle(case):
    hidden, group, fmt, sfmt = case
    say("cast fp32", case)
    base = wl.WORKLOADS["fp8_g128_fp32_ragged_h7168"]
    rows = 61
    xs = wl.make_x(base, 2, rows=range(rows))
    x = np.ascontiguousarray(np.tile(xs, (1, (2 * hidden + xs.shape[1] - 1) // xs.shape[1]))[:, :2 * hidden])
    wt = wl.make_w(base, 2)[:rows] if wl.num_rows(base, 2) >= rows else None
    y, _ = oracle.swiglu_forward(x, wt, None)
    y[3, :] = 0.0
    y[5, 1::3] = np.float32(1e-42)  # subnormals
    yd = torch.from_numpy(y).to(DEV)
    got = run_cast(yd, tk.TK_DTYPE_FP32, rows, hidden, group, fmt, sfmt)
    same(got, oracle.cast(y, group, fmt, sfmt), f"fp32 {case}")


@pytest.mark.parametrize("fmt", [8, 4])
def test_converter_sweep_through_the_abi(fmt):
    """Every 5th fp32 bit pattern with |q| <= fmt_max, both signs, cast with
    scale exactly 1 (each row holds one element equal to fmt_max): the gfx950
    converters against the oracle's codec, including ties and subnormals."""
    fmt_max = 448.0 if fmt == 8 else 6.0
    hi = int(np.float32(fmt_max).view(np.uint32))
    bits = np.arange(0, hi + 1, 5, dtype=np.uint32)
    vals = bits.view(np.float32)
    vals = np.concatenate([vals, -vals])
    hidden = 8192
    per_row = hidden - 8
    rows = (len(vals) + per_row - 1) // per_row
    say("converter sweep", fmt, "values", len(vals), "rows", rows)
    y = np.zeros((rows, hidden), dtype=np.float32)
    flat = y[:, 8:].reshape(-1)
    flat[:len(vals)] = vals
    y[:, 8:] = flat.reshape(rows, per_row)
    y[:, 0] = fmt_max
    yd = torch.from_numpy(y).to(DEV)
    for sfmt in (tk.TK_SCALE_UE8M0, tk.TK_SCALE_FP32):
        codes, scales = run_cast(yd, tk.TK_DTYPE_FP32, rows, hidden, 0, fmt, sfmt)
        if sfmt == tk.TK_SCALE_UE8M0:
            assert (scales == 127).all()
        else:
            assert (scales == 1.0).all()
        want = oracle.encode(y, fmt)
        if fmt == 4:
            want = (want[:, 0::2] | (want[:, 1::2] << 4)).astype(np.uint8)
        assert np.array_equal(codes, want), np.argwhere(codes != want)[:5]


@pytest.mark.parametrize("name", ["fp8_g128_ue8m0_n32768_h2048", "fp8_per_token_clamp10_n131072_h2048",
                                  "fp4_g32_ue8m0_n65536_h4096", "fp8_g128_fp32_ragged_h7168"])
def test_unfused_two_kernel_path_equals_fused(name):
    """tk_swiglu_forward (fp32 y) then tk_cast (fp32 in) gives exactly the fused
    kernel's codes, scales and clamp count, on every row at full size."""
    w = wl.WORKLOADS[name]
    n = wl.num_rows(w, 0)
    say("unfused == fused", name, n)
    x, wt = wl.make_x(w, 0), wl.make_w(w, 0)
    fmt = 8 if w.fmt == "fp8" else 4
    sfmt = tk.TK_SCALE_FP32 if w.scale_fmt == "fp32" else tk.TK_SCALE_UE8M0
    clamp = math.inf if w.clamp_limit is None else w.clamp_limit
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    wd = torch.from_numpy(wt).to(DEV)
    del x
    y = torch.empty((n, w.hidden), dtype=torch.float32, device=DEV)
    c1 = torch.zeros(1, dtype=torch.int64, device=DEV)
    assert tk.tk_swiglu_forward(xd, wd, n, w.hidden, clamp, y, c1) == OK
    unfused = run_cast(y, tk.TK_DTYPE_FP32, n, w.hidden, w.group_size, fmt, sfmt)
    del y
    codes = torch.empty((n, w.code_bytes_per_row), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, w.groups_per_row * (4 if sfmt == 0 else 1)), dtype=torch.uint8, device=DEV)
    c2 = torch.zeros(1, dtype=torch.int64, device=DEV)
    fn = tk.tk_swiglu_cast_fp8 if fmt == 8 else tk.tk_swiglu_cast_fp4
    assert fn(xd, wd, n, w.hidden, w.group_size, clamp, sfmt, codes, scales, c2) == OK
    torch.cuda.synchronize()
    fused_scales = scales.cpu().numpy()
    fused_scales = fused_scales.view(np.float32) if sfmt == 0 else fused_scales
    same(unfused, (codes.cpu().numpy(), fused_scales), name)
    assert int(c1.item()) == int(c2.item())


def test_benchmark_workload_full_size_every_row():
    """The stand-alone cast exactly as the benchmark times it: bf16 rows
    [65536, 2048] (the N(0,2) samples of a [32768, 4096] draw), groups of 128,
    UE8M0 scales; every code and scale against the oracle."""
    n, hidden, group = 32768, 2048, 128
    w = wl.Workload("cast_bf16_e4m3_g128_ue8m0_n65536_h2048", n, hidden, 2.0, "fp8", group, "ue8m0", None, "uniform")
    say("cast benchmark workload, full size")
    x = wl.make_x(w, 0).reshape(2 * n, hidden)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    got = run_cast(xd, tk.TK_DTYPE_BF16, 2 * n, hidden, group, 8, tk.TK_SCALE_UE8M0)
    same(got, oracle.cast_bf16(x, group, 8, tk.TK_SCALE_UE8M0), "cast benchmark workload")
