"""GPU parity of row-reduced groups longer than one wave holds (per-token rows
and column groups beyond 8192 columns, up to 32768): 2 or 4 waves of a
workgroup share one group and meet in LDS for its abs-max.  Fused and
stand-alone cast paths, FP8 and FP4, fp32 and UE8M0 scales, with and without
the clamp, against the oracle bit for bit.

Each case plants, row by row, the group's largest value in a different
wave's share (at that share's last column, the row's last column for the
ragged share), so a wave that quantised with its own abs-max instead of the
group's would get the scale wrong (with the clamp on, the planted value is
clamped to the ceiling and may tie with others)."""
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
FP32, UE8M0 = tk.TK_SCALE_FP32, tk.TK_SCALE_UE8M0
BF16 = {256.0: 0x4380, 4096.0: 0x4580, -4096.0: 0xC580}  # the inputs stay within |50|


def say(*a):
    print("[gpu-case]", *a, flush=True)


def share_ends(hidden, group):
    """Last column of every wave's share of every group: the split the library
    documents (2 waves up to 32 steps of 512 columns, else 4; ceil(k/W) steps
    each, the last share shorter)."""
    G = hidden if group == 0 else group
    k = -(-(G // 8) // 64)
    waves = 2 if k <= 32 else 4
    spw = -(-k // waves)
    ends = []
    for g0 in range(0, hidden, G):
        for part in range(waves):
            ends.append(min(g0 + (part + 1) * spw * 512, g0 + G) - 1)
    return ends


def inputs(n, hidden, seed):
    base = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    full = wl.make_x(base, seed, rows=range(n))
    return np.ascontiguousarray(np.tile(full, (1, (2 * hidden + 4095) // 4096))[:, :2 * hidden])


def plant_swiglu(x, hidden, group):
    ends = share_ends(hidden, group)
    for r in range(x.shape[0]):
        c = ends[r % len(ends)]
        x[r, c] = BF16[256.0]
        x[r, hidden + c] = BF16[256.0]


def plant_cast(x, hidden, group):
    ends = share_ends(hidden, group)
    for r in range(x.shape[0]):
        x[r, ends[r % len(ends)]] = BF16[4096.0 if r % 3 else -4096.0]


def bufs(n, hidden, group, fmt, sfmt):
    groups = 1 if group == 0 else hidden // group
    cols = hidden if fmt == 8 else hidden // 2
    sitem = 4 if sfmt == FP32 else 1
    cbuf = torch.full((n * cols + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((n * groups * sitem + 2 * PAD,), 0x5A, dtype=torch.uint8, device=DEV)
    return cbuf, sbuf, cols, groups, sitem


def fetch(cbuf, sbuf, n, cols, groups, sitem):
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (c[:PAD] == 0xA5).all() and (c[len(c) - PAD:] == 0xA5).all(), "codes canary overwritten"
    assert (s[:PAD] == 0x5A).all() and (s[len(s) - PAD:] == 0x5A).all(), "scales canary overwritten"
    sb = s[PAD:len(s) - PAD]
    return c[PAD:len(c) - PAD].reshape(n, cols), (sb.view(np.float32) if sitem == 4 else sb).reshape(n, groups)


def same(got, want, what):
    (gc, gs), (wc, ws) = got, want
    if not np.array_equal(gs.view(np.uint8), ws.view(np.uint8)):
        bad = np.argwhere(gs.view(np.uint8).reshape(gs.shape[0], -1) != ws.view(np.uint8).reshape(ws.shape[0], -1))
        raise AssertionError(f"{what}: scales differ at {bad[:5].tolist()}")
    if not np.array_equal(gc, wc):
        bad = np.argwhere(gc != wc)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first row {r} col {c}")


CASES = [  # (rows, hidden, group, fmt, scale, clamp)
    (21, 8200, 0, 8, FP32, None),        # 17 steps: 2 waves of 9 + 8, ragged last step
    (13, 10000, 0, 4, UE8M0, 10.0),      # 20 steps, ragged
    (9, 14336, 0, 8, UE8M0, None),       # 28 steps
    (11, 16384, 0, 8, FP32, 10.0),       # 32 steps: 2 waves of 16
    (7, 16392, 0, 8, FP32, None),        # 33 steps: 4 waves of 9, 9, 9, 6, ragged
    (6, 24576, 0, 4, FP32, None),        # 48 steps
    (5, 32768, 0, 8, UE8M0, 2.0),        # 64 steps: 4 waves of 16
    (5, 32768, 16384, 8, FP32, None),    # two groups of 32 steps
    (3, 36864, 18432, 4, UE8M0, None),   # two groups of 36 steps: 4 waves of 9
    (6, 17408, 17408, 8, FP32, None),    # one group of 34 steps: 9, 9, 9, 7
    (7, 26624, 13312, 8, UE8M0, 10.0),   # two groups of 26 steps
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_fused_long_groups(case):
    n, hidden, group, fmt, sfmt, clamp = case
    say("fused long group", case)
    x = inputs(n, hidden, 5)
    plant_swiglu(x, hidden, group)
    wt = wl.make_w(wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"], 5)[:n]
    cbuf, sbuf, cols, groups, sitem = bufs(n, hidden, group, fmt, sfmt)
    cnt = torch.zeros(3, dtype=torch.int64, device=DEV)
    fn = tk.tk_swiglu_cast_fp8 if fmt == 8 else tk.tk_swiglu_cast_fp4
    rc = fn(torch.from_numpy(x.view(np.int16)).to(DEV), torch.from_numpy(wt).to(DEV), n, hidden, group,
            math.inf if clamp is None else clamp, sfmt, cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD,
            cnt.data_ptr() + 8)
    assert rc == OK, tk.tk_status_str(rc)
    got = fetch(cbuf, sbuf, n, cols, groups, sitem)
    wc, ws, wk = oracle.swiglu_cast(x, wt, group, clamp, fmt, sfmt)
    same(got, (wc, ws), f"fused {case}")
    k = cnt.cpu().numpy()
    assert k[0] == 0 and k[2] == 0 and k[1] == wk
    if clamp is not None:
        assert wk > 0


@pytest.mark.parametrize("case", CASES, ids=str)
@pytest.mark.parametrize("in_dtype", ["bf16", "fp32"])
def test_cast_long_groups(case, in_dtype):
    n, hidden, group, fmt, sfmt, _ = case
    say("cast long group", in_dtype, case)
    if in_dtype == "bf16":
        x = np.ascontiguousarray(inputs(n, hidden, 6)[:, :hidden])
        plant_cast(x, hidden, group)
        xd = torch.from_numpy(x.view(np.int16)).to(DEV)
        want = oracle.cast_bf16(x, group, fmt, sfmt)
        dt = tk.TK_DTYPE_BF16
    else:
        x = inputs(n, hidden, 6)
        plant_swiglu(x, hidden, group)
        y, _ = oracle.swiglu_forward(x, None, None)
        y[n // 2, ::7] = np.float32(1e-42)  # subnormals
        xd = torch.from_numpy(y).to(DEV)
        want = oracle.cast(y, group, fmt, sfmt)
        dt = tk.TK_DTYPE_FP32
    cbuf, sbuf, cols, groups, sitem = bufs(n, hidden, group, fmt, sfmt)
    fn = tk.tk_cast_fp8 if fmt == 8 else tk.tk_cast_fp4
    rc = fn(xd, dt, n, hidden, group, sfmt, cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD)
    assert rc == OK, tk.tk_status_str(rc)
    same(fetch(cbuf, sbuf, n, cols, groups, sitem), want, f"cast {in_dtype} {case}")


def sample_rows(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(24), np.arange(n - 24, n), rng.choice(n, 48, replace=False)]))


def test_fused_long_rows_many_passes():
    """3001 rows of 8200 columns: more groups than the grid holds, so every
    workgroup runs several passes (the double-buffered maxes); codes and
    scales of sampled rows against the oracle."""
    n, hidden = 3001, 8200
    say("fused long rows, passes", n, hidden)
    x = inputs(n, hidden, 8)
    plant_swiglu(x, hidden, 0)
    wt = wl.make_w(wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"], 8)[:n]
    cbuf, sbuf, cols, groups, sitem = bufs(n, hidden, 0, 8, FP32)
    rc = tk.tk_swiglu_cast_fp8(torch.from_numpy(x.view(np.int16)).to(DEV), torch.from_numpy(wt).to(DEV), n, hidden,
                               0, math.inf, FP32, cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD, None)
    assert rc == OK
    gc, gs = fetch(cbuf, sbuf, n, cols, groups, sitem)
    rows = sample_rows(n, 1)
    wc, ws, _ = oracle.swiglu_cast(x[rows], wt[rows], 0, None, 8, FP32)
    same((gc[rows], gs[rows]), (wc, ws), "fused passes")


def test_cast_long_rows_many_passes():
    """4501 bf16 rows of 8200 columns through the stand-alone cast: past its
    grid cap, so workgroups loop over passes; sampled rows against the oracle."""
    n, hidden = 4501, 8200
    say("cast long rows, passes", n, hidden)
    x = np.ascontiguousarray(inputs(n, hidden, 9)[:, :hidden])
    plant_cast(x, hidden, 0)
    cbuf, sbuf, cols, groups, sitem = bufs(n, hidden, 0, 4, UE8M0)
    rc = tk.tk_cast_fp4(torch.from_numpy(x.view(np.int16)).to(DEV), tk.TK_DTYPE_BF16, n, hidden, 0, UE8M0,
                        cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD)
    assert rc == OK
    gc, gs = fetch(cbuf, sbuf, n, cols, groups, sitem)
    rows = sample_rows(n, 2)
    same((gc[rows], gs[rows]), oracle.cast_bf16(x[rows], 0, 4, UE8M0), "cast passes")
