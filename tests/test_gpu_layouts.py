"""GPU parity of the column-major and packed scale layouts, on the fused and
the stand-alone cast paths: codes as in the row-major case, scales at the
layout's positions, bytes the layout leaves unwritten untouched."""
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
LAYOUTS = {tk.TK_SCALE_FP32_COLMAJOR: ("fp32_colmajor", 0), tk.TK_SCALE_UE8M0_COLMAJOR: ("ue8m0_colmajor", 1),
           tk.TK_SCALE_UE8M0_PACKED: ("ue8m0_packed", 1)}
CASES = [  # (rows, hidden, group, fmt, clamp)
    (37, 2048, 128, 8, None), (21, 4096, 32, 4, None), (13, 2048, 0, 8, 10.0), (70, 7168, 128, 8, None),
    (9, 1024, 512, 4, 2.0), (50, 1000, 8, 8, None),
    (5, 32768, 16384, 8, None), (6, 10000, 0, 4, 10.0),  # groups shared by several waves
]


def layout_bytes(name, n, groups):
    if name == "fp32_colmajor":
        return groups * ((n + 3) // 4 * 4) * 4
    if name == "ue8m0_colmajor":
        return groups * ((n + 15) // 16 * 16)
    return (groups + 3) // 4 * ((n + 3) // 4 * 4) * 4


@pytest.mark.parametrize("path", ["fused", "cast"])
@pytest.mark.parametrize("sfmt", list(LAYOUTS))
@pytest.mark.parametrize("case", CASES, ids=str)
def test_scale_layout(case, sfmt, path):
    n, hidden, group, fmt, clamp = case
    name, kind = LAYOUTS[sfmt]
    print("[gpu-case] layout", case, name, path, flush=True)
    base = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    full = wl.make_x(base, 7, rows=range(n))
    x = np.ascontiguousarray(np.tile(full, (1, (2 * hidden + 4095) // 4096))[:, :2 * hidden])
    wt = wl.make_w(base, 7)[:n]
    groups = 1 if group == 0 else hidden // group
    cols = hidden if fmt == 8 else hidden // 2
    nbytes = layout_bytes(name, n, groups)
    cbuf = torch.full((n * cols + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((nbytes + 2 * PAD,), 0xFF, dtype=torch.uint8, device=DEV)
    if path == "fused":
        xd = torch.from_numpy(x.view(np.int16)).to(DEV)
        wd = torch.from_numpy(wt).to(DEV)
        fn = tk.tk_swiglu_cast_fp8 if fmt == 8 else tk.tk_swiglu_cast_fp4
        rc = fn(xd, wd, n, hidden, group, math.inf if clamp is None else clamp, sfmt, cbuf.data_ptr() + PAD,
                sbuf.data_ptr() + PAD, None)
        want_codes, want_scales, _ = oracle.swiglu_cast(x, wt, group, clamp, fmt, kind)
    else:
        y, _ = oracle.swiglu_forward(x, wt, clamp)
        yd = torch.from_numpy(y).to(DEV)
        fn = tk.tk_cast_fp8 if fmt == 8 else tk.tk_cast_fp4
        rc = fn(yd, tk.TK_DTYPE_FP32, n, hidden, group, sfmt, cbuf.data_ptr() + PAD, sbuf.data_ptr() + PAD)
        want_codes, want_scales = oracle.cast(y, group, fmt, kind)
    assert rc == tk.TkStatus.TK_OK, tk.tk_status_str(rc)
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (c[:PAD] == 0xA5).all() and (c[-PAD:] == 0xA5).all()
    assert (s[:PAD] == 0xFF).all() and (s[-PAD:] == 0xFF).all()
    assert np.array_equal(c[PAD:-PAD].reshape(n, cols), want_codes)
    want = oracle.scale_layout(want_scales, name, 0xFF)
    got = s[PAD:-PAD]
    assert got.shape == want.shape
    assert np.array_equal(got, want), np.argwhere(got != want)[:8].ravel()
