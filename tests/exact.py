"""Exact-arithmetic brute-force evaluator used to pin the oracle.

Independent of oracle/oracle.c by construction: every fp32 rounding is done
on exact rationals (fractions.Fraction) by counting ulps, the sigmoid is taken
in 60-digit decimal arithmetic, codes are found by searching the whole code
table for the nearest value (ties to the even code, the largest finite code
for anything beyond it), and the UE8M0 exponent is the ceiling of an exact
base-2 logarithm.  It is slow and only meant for tiny inputs.
"""
from __future__ import annotations

import math
import struct
from decimal import Decimal, getcontext
from fractions import Fraction as Fr
from typing import List, Optional, Sequence, Tuple

getcontext().prec = 60

FLT_MAX = Fr((2 ** 24 - 1) * 2 ** 104)


def bf16_to_float(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (h & 0xFFFF) << 16))[0]


def float_to_bf16(f: float) -> int:
    """Exact bf16 bit pattern of a value that is representable in bf16."""
    b = struct.unpack("<I", struct.pack("<f", f))[0]
    assert b & 0xFFFF == 0, f"{f} is not a bf16 value"
    return b >> 16


def is_neg(v: float) -> bool:
    return math.copysign(1.0, v) < 0


def round_f32(x: Fr, neg_zero: bool = False) -> float:
    """Round an exact rational to fp32, nearest-even, with subnormals and overflow to inf."""
    if x == 0:
        return -0.0 if neg_zero else 0.0
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fr(2) ** (e - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    m = n * ulp
    if m >= Fr(2) ** 128:
        r = math.inf
    else:
        r = float(m)  # exact: m has at most 24 significant bits
    if r == 0.0:
        return -0.0 if neg else 0.0
    return -r if neg else r


def mul_f32(a: float, b: float) -> float:
    return round_f32(Fr(a) * Fr(b), neg_zero=is_neg(a) != is_neg(b))


def div_f32(a: float, b: float) -> float:
    if b == 0:
        return math.inf if a >= 0 else -math.inf
    return round_f32(Fr(a) / Fr(b), neg_zero=is_neg(a) != is_neg(b))


def sigmoid_f32(g: float) -> float:
    """Correctly rounded fp32 of 1/(1+e^-g) from 60-digit decimal arithmetic."""
    if g >= 40.0:
        return 1.0  # 1 - sigma < e^-40, far below half an ulp of 1
    if g <= -200.0:
        return 0.0  # sigma < e^-200 < 2^-288
    s = Decimal(1) / (Decimal(1) + (-Decimal(g)).exp())
    return round_f32(Fr(s))


def e4m3_values() -> List[Fr]:
    vals = []
    for c in range(127):  # 0x00..0x7E: the finite non-negative codes
        e, m = c >> 3, c & 7
        vals.append(Fr(m, 8) * Fr(2) ** -6 if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7))
    return vals


def e2m1_values() -> List[Fr]:
    return [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


E4M3 = e4m3_values()
E2M1 = e2m1_values()


def nearest_code(q: float, table: Sequence[Fr], sign_bit: int) -> int:
    """Nearest table entry to |q| (ties -> even code), sign bit from q."""
    a = abs(Fr(q))
    best, best_d = 0, None
    for c, v in enumerate(table):
        d = abs(v - a)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (sign_bit if is_neg(q) else 0)


def decode(code: int, fmt: int) -> Fr:
    if fmt == 8:
        v = E4M3[code & 0x7F]
        return -v if code & 0x80 else v
    v = E2M1[code & 0x7]
    return -v if code & 0x8 else v


def ue8m0_k(amax: float, fmt_max: float) -> int:
    """Smallest k >= -127 with fmt_max * 2^k >= amax, via an exact ceil(log2)."""
    if amax == 0:
        return -127
    r = Fr(amax) / Fr(fmt_max)
    k = r.numerator.bit_length() - r.denominator.bit_length()
    while Fr(2) ** k < r:
        k += 1
    while Fr(2) ** (k - 1) >= r:
        k -= 1
    return max(k, -127)


def swiglu_row(gate: Sequence[int], up: Sequence[int], w: Optional[float],
               clamp: Optional[float]) -> Tuple[List[float], int]:
    """fp32 y of one row from bf16 bit patterns, and its clamp count."""
    y, count = [], 0
    for gh, uh in zip(gate, up):
        g, u = bf16_to_float(gh), bf16_to_float(uh)
        if clamp is not None:
            if g > clamp:
                g = clamp
                count += 1
            u = min(max(u, -clamp), clamp)
        a = mul_f32(g, sigmoid_f32(g))
        b = mul_f32(a, u)
        y.append(b if w is None else mul_f32(b, w))
    return y, count


def cast_row(y: Sequence[float], group: int, fmt: int, scale_fmt: int):
    """(codes one per element, scales) of one fp32 row."""
    fmt_max = 448.0 if fmt == 8 else 6.0
    table, sign = (E4M3, 0x80) if fmt == 8 else (E2M1, 0x8)
    G = group or len(y)
    codes, scales = [], []
    for k0 in range(0, len(y), G):
        grp = y[k0:k0 + G]
        amax = max(abs(v) for v in grp)
        if scale_fmt == 0:
            scales.append(div_f32(amax, fmt_max))
            inv = div_f32(fmt_max, amax)
            inv = min(inv, float(FLT_MAX))
        else:
            k = ue8m0_k(amax, fmt_max)
            scales.append(k + 127)
            inv = float(Fr(2) ** -k)
        for v in grp:
            codes.append(nearest_code(mul_f32(v, inv), table, sign))
    return codes, scales


def pack_fp4(codes: Sequence[int]) -> List[int]:
    return [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)]


def add_f32(a: float, b: float) -> float:
    """RN(a + b) in fp32; an exact zero sum is +0 unless both addends are -0."""
    s = Fr(a) + Fr(b)
    return round_f32(s, neg_zero=(s == 0 and is_neg(a) and is_neg(b)))


def round_bf16(v: float) -> int:
    """bf16 bit pattern nearest to the finite value v, ties to the even code,
    found by searching the neighbouring codes on exact rationals."""
    if v == 0:
        return 0x8000 if is_neg(v) else 0
    best, best_d = None, None
    b = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    for code in range(max(0, (b & 0x7FFF) - 2), min(0x7F80, (b & 0x7FFF) + 3) + 1):
        mag = Fr(2) ** 128 if code == 0x7F80 else Fr(bf16_to_float(code))
        d = abs(abs(Fr(v)) - mag)
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best | (b & 0x8000)


def reduce_cell(xs: Sequence[int], ws: Sequence[float], scales: Sequence[Optional[float]], gscale: float) -> float:
    """One output element of the weighted top-k reduce over the present slots,
    in slot order: f = RN(w*s), acc = RN(acc + RN(f*x)) from +0, then
    RN(acc*gscale)."""
    acc = 0.0
    for xh, w, s in zip(xs, ws, scales):
        f = w if s is None else mul_f32(w, s)
        acc = add_f32(acc, mul_f32(f, bf16_to_float(xh)))
    return mul_f32(acc, gscale)
