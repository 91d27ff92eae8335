"""GPU parity on a seeded random sweep of the parameters of the fused step
(tk_swiglu_cast_fp8/fp4), the stand-alone cast (tk_cast_fp8/fp4) and the
weighted top-k reduce (tk_moe_reduce) against the oracle, bit-exact.

Each case draws its rows (1 .. 300), width (multiples of 8 from 8 to 8192,
with and without a partial last 512-column step), group (per-token or any
multiple of 8 dividing the width), code format, scale kind, clamp limit (off, or 0.5
to 1e4), routing weights (none; U(0,1) with a fifth exactly 0; some negative)
and a per-row input magnitude from 1e-20 to 1e6.  The 1e-20 rows make
subnormal fp32 products, so UE8M0 exponents reach their floor of -127 and
fp32 scales go subnormal; the 1e6 rows keep every product finite.  Inputs come
from numpy's seeded generator, rounded to bf16 to nearest even."""
import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
import oracle
from test_gpu_cast import run_cast as run_standalone_cast
from test_gpu_cast import same as same_cast
from test_gpu_parity import DEV, assert_same, run_cast, say

pytestmark = pytest.mark.gpu

HIDDENS = [8, 16, 24, 64, 136, 512, 520, 1024, 1032, 2048, 3072, 4104, 7168, 8192]
ROWS = [1, 2, 63, 64, 65, 129, 300]
MAGNITUDES = [1e-20, 1e-6, 1.0, 100.0, 1e6]


def bf16_bits(f):
    """fp32 values to bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def draw(i, cols_factor):
    rng = np.random.default_rng(20_000 + 97 * i + cols_factor)
    fmt = int(rng.choice([8, 4]))
    hidden = int(rng.choice(HIDDENS))
    groups = [0] + [g for g in range(8, hidden + 1, 8) if hidden % g == 0]
    group = int(rng.choice(groups))
    sfmt = int(rng.choice([tk.TK_SCALE_FP32, tk.TK_SCALE_UE8M0]))
    clamp = None if rng.random() < 0.5 else float(rng.choice([0.5, 3.0, 10.0, 1e4]))
    n = int(rng.choice(ROWS))
    mag = rng.choice(MAGNITUDES, size=(n, 1))
    x = bf16_bits(rng.standard_normal((n, cols_factor * hidden)) * mag)
    w = None
    if rng.random() < 0.7:
        w = rng.uniform(0.0, 1.0, n).astype(np.float32)
        w[rng.random(n) < 0.2] = 0.0
        if rng.random() < 0.2:
            w[::3] = -w[::3]
    return fmt, hidden, group, sfmt, clamp, n, x, w


@pytest.mark.parametrize("i", range(64))
def test_random_fused_case(i):
    fmt, hidden, group, sfmt, clamp, n, x, w = draw(i, 2)
    say("random fused", i, dict(fmt=fmt, hidden=hidden, group=group, sfmt=sfmt, clamp=clamp, n=n,
                                weighted=w is not None))
    got = run_cast(x, w, hidden, group, clamp, fmt, sfmt)
    want = oracle.swiglu_cast(x, w, group, clamp, fmt, sfmt)
    assert_same(got, want, f"random fused case {i}")


@pytest.mark.parametrize("i", range(32))
def test_random_standalone_cast_case(i):
    fmt, hidden, group, sfmt, _, n, x, _ = draw(i, 1)
    say("random cast", i, dict(fmt=fmt, hidden=hidden, group=group, sfmt=sfmt, n=n))
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    got = run_standalone_cast(xd, tk.TK_DTYPE_BF16, n, hidden, group, fmt, sfmt)
    same_cast(got, oracle.cast_bf16(x, group, fmt, sfmt), f"random cast case {i}")


@pytest.mark.parametrize("i", range(32))
def test_random_reduce_case(i):
    """tk_moe_reduce on a random draw: tokens, k (1 .. 64), width, position
    map with repeated rows, dropped (-1) and out-of-range entries, weights
    with zeros and negatives, optional per-row scales, global scale of
    either sign and tiny magnitude, bf16 or fp32 output."""
    from test_gpu_reduce import run_reduce, same as same_reduce
    rng = np.random.default_rng(30_000 + i)
    tokens = int(rng.choice([1, 7, 64, 200]))
    k = int(rng.choice([1, 2, 3, 5, 8, 9, 12, 16, 24, 32, 40, 64]))
    hidden = int(rng.choice([8, 24, 64, 520, 1024, 2056, 7168]))
    n_rows = int(rng.integers(1, 3 * tokens * k // 2 + 2))
    pos = rng.integers(0, n_rows, size=(tokens, k)).astype(np.int32)
    pos[rng.random((tokens, k)) < 0.1] = -1
    pos[rng.random((tokens, k)) < 0.03] = n_rows + 5
    w = rng.uniform(-0.25, 1.0, (tokens, k)).astype(np.float32)
    w[rng.random((tokens, k)) < 0.1] = 0.0
    rs = rng.uniform(0.5, 2.0, n_rows).astype(np.float32) if rng.random() < 0.5 else None
    gs = float(rng.choice([1.0, 2.5, -0.75, 1e-30]))
    out_bf16 = bool(rng.random() < 0.6)
    mag = rng.choice(MAGNITUDES, size=(n_rows, 1))
    x = bf16_bits(rng.standard_normal((n_rows, hidden)) * mag)
    say("random reduce", i, dict(tokens=tokens, k=k, hidden=hidden, n_rows=n_rows, scaled=rs is not None, gs=gs,
                                 bf16=out_bf16))
    got = run_reduce(x, pos, w, rs, gs, out_bf16)
    same_reduce(got, oracle.moe_reduce(x, pos, w, rs, gs, out_bf16), f"random reduce case {i}")
