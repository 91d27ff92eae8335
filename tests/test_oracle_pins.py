"""Pins of the oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
rows (tests/golden), an exact-rational brute-force evaluator (tests/exact.py),
a library routine (torch's float8_e4m3fn cast), 60-digit decimal arithmetic,
closed forms and invariants.
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import exact as E
import oracle
from moe_activation_bit_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")


def _row_x(gate, up):
    return np.array([[E.float_to_bf16(v) for v in gate] + [E.float_to_bf16(v) for v in up]], dtype=np.uint16)


def _hand_rows():
    return json.load(open(GOLDEN))["rows"]


@pytest.mark.parametrize("row", _hand_rows(), ids=lambda r: r["name"])
def test_hand_rows_oracle(row):
    x = _row_x(row["gate"], row["up"])
    w = np.array([row["weight"]], dtype=np.float32)
    codes, scales, cnt = oracle.swiglu_cast(x, w, row["group"], row["clamp"], row["fmt"], row["scale_fmt"])
    assert codes[0].tolist() == row["codes"]
    if row["scale_fmt"] == 0:
        assert scales[0].tolist() == row["scales_f32"]
    else:
        assert scales[0].tolist() == row["scales_u8"]
    assert cnt == row["count"]
    if "y" in row:
        y, cnt2 = oracle.swiglu_forward(x, w, row["clamp"])
        assert [float(v) for v in y[0]] == row["y"]
        assert [math.copysign(1, v) for v in y[0]] == [math.copysign(1, v) for v in row["y"]]
        assert cnt2 == row["count"]


@pytest.mark.parametrize("row", _hand_rows(), ids=lambda r: r["name"])
def test_hand_rows_exact_evaluator(row):
    gh = [E.float_to_bf16(v) for v in row["gate"]]
    uh = [E.float_to_bf16(v) for v in row["up"]]
    y, cnt = E.swiglu_row(gh, uh, row["weight"], row["clamp"])
    codes, scales = E.cast_row(y, row["group"], row["fmt"], row["scale_fmt"])
    if row["fmt"] == 4:
        codes = E.pack_fp4(codes)
    assert codes == row["codes"]
    assert scales == (row["scales_f32"] if row["scale_fmt"] == 0 else row["scales_u8"])
    assert cnt == row["count"]


def test_sigmoid_exhaustive_bf16():
    """sigma(g) for every finite bf16 g equals the correctly rounded fp32 of 1/(1+e^-g)."""
    h = np.arange(65536, dtype=np.uint32)
    g = (h << 16).view(np.float32)
    bad = []
    for v in g[np.isfinite(g)]:
        v = float(v)
        got = oracle.sigmoid(v)
        want = E.sigmoid_f32(v)
        if np.float32(got).view(np.uint32) != np.float32(want).view(np.uint32):
            bad.append((v, got, want))
    assert not bad, bad[:10]


def test_sigmoid_random_fp32():
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.uniform(-30, 30, 600), rng.standard_normal(300) * 1e-4,
                           [10.0, 2.5, 7.75, 1e-30, -1e-30, 17.3, 17.4, -103.9, -104.1]]).astype(np.float32)
    for v in vals:
        assert oracle.sigmoid(float(v)) == E.sigmoid_f32(float(v)), float(v)


def _f32_sweep(lo_bits, hi_bits, stride, offset=0):
    return np.arange(lo_bits + offset, hi_bits, stride, dtype=np.uint32).view(np.float32)


def test_e4m3_matches_torch_cast_sweep():
    """Library routine: torch's float8_e4m3fn cast is round-to-nearest-even and
    agrees with a saturating cast wherever no saturation happens (|q| <= 448)."""
    torch = pytest.importorskip("torch")
    hi = np.float32(448.0).view(np.uint32)
    for off in (0, 5):
        q = _f32_sweep(0, int(hi) + 1, 13, off)
        for chunk in np.array_split(q, 8):
            for sgn in (1.0, -1.0):
                c = (chunk * np.float32(sgn)).astype(np.float32)
                ref = torch.from_numpy(c).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                got = oracle.encode(c, 8)
                mism = np.nonzero(ref != got)[0]
                assert mism.size == 0, [(float(c[i]), got[i], ref[i]) for i in mism[:5]]


def test_e4m3_saturates():
    q = np.array([448.0, 448.00003, 463.99997, 464.0, 464.00003, 480.0, 1e6, 3.4e38], dtype=np.float32)
    for s in (1, -1):
        got = oracle.encode(q * s, 8)
        assert (got == (0x7E if s > 0 else 0xFE)).all(), got


def _neighbours(v, k):
    b = int(np.float32(v).view(np.uint32))
    return [np.uint32(b + d).view(np.float32) for d in range(-k, k + 1) if 0 <= b + d]


def test_e4m3_brute_force_at_every_midpoint():
    vals = E.E4M3
    pts = []
    for c in range(126):
        mid = (vals[c] + vals[c + 1]) / 2
        pts += _neighbours(np.float32(float(mid)), 3)
        pts += _neighbours(np.float32(float(vals[c])), 1)
    pts += [np.float32(v) for v in (0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -149, 440.0, 447.9, 456.0)]
    for p in pts:
        for s in (1.0, -1.0):
            q = float(np.float32(p) * np.float32(s))
            assert oracle.e4m3(q) == E.nearest_code(q, E.E4M3, 0x80), q
    assert oracle.e4m3(-0.0) == 0x80 and oracle.e4m3(0.0) == 0x00


def test_e2m1_brute_force_sweep():
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    hi = int(np.float32(8.0).view(np.uint32))
    q = _f32_sweep(0, hi, 101)  # every binade up to 8 (the midpoints have a test of their own)
    for chunk in np.array_split(q, 4):
        a = chunk.astype(np.float64)
        d = np.abs(a[:, None] - vals[None, :])
        first = d.argmin(1)
        last = 7 - d[:, ::-1].argmin(1)
        want = np.where(first % 2 == 0, first, last).astype(np.uint8)
        assert np.array_equal(oracle.encode(chunk, 4), want)
        assert np.array_equal(oracle.encode(-chunk, 4), want | 0x8)


def test_e2m1_ties():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7}
    for v, c in ties.items():
        assert oracle.e2m1(v) == c and oracle.e2m1(-v) == c | 8


def _ue8m0_points(fmt_max):
    pts = [0.0, 2.0 ** -149, 2.0 ** -126, 1e-38, 3.4e38, float(np.finfo(np.float32).max)]
    for k in range(-127, 121):
        v = np.float32(fmt_max * 2.0 ** k)
        if np.isfinite(v) and v > 0:
            pts += [float(x) for x in _neighbours(v, 1)]
    rng = np.random.default_rng(3)
    pts += list((2.0 ** rng.uniform(-140, 127, 400)).astype(np.float32).astype(float))
    return [p for p in pts if np.isfinite(np.float32(p))]


@pytest.mark.parametrize("fmt", [8, 4])
def test_ue8m0_closed_form(fmt):
    fmt_max = 448.0 if fmt == 8 else 6.0
    for amax in _ue8m0_points(fmt_max):
        amax = float(np.float32(amax))
        k = oracle.ue8m0_exponent(amax, fmt)
        assert Fr(fmt_max) * Fr(2) ** k >= Fr(amax), (amax, k)
        if k > -127:
            assert Fr(fmt_max) * Fr(2) ** (k - 1) < Fr(amax), (amax, k)
        assert k == E.ue8m0_k(amax, fmt_max)


CASES = [  # (hidden, group, fmt, scale_fmt, clamp)
    (16, 0, 8, 0, None), (16, 8, 8, 1, None), (16, 0, 4, 1, 2.5), (16, 8, 4, 0, None),
    (24, 8, 8, 0, 1.0), (8, 0, 8, 1, 0.75), (16, 4, 4, 1, None), (32, 16, 8, 0, 3.0),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_oracle_matches_exact_evaluator_on_tiny_rows(case):
    hidden, group, fmt, sfmt, clamp = case
    base = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    rng = np.random.default_rng(hidden * 31 + group)
    rows = 6
    x = np.empty((rows, 2 * hidden), dtype=np.uint16)
    for r in range(rows):
        full = wl.make_x(base, r, rows=[r])[0]
        x[r] = full[: 2 * hidden]
    # exact ties and specials: a gate exactly at the limit, signed zeros, big values
    x[0, 0] = E.float_to_bf16(clamp if clamp is not None else 1.0)
    x[1, 1] = 0x8000
    x[1, hidden] = 0x8000
    x[2, 2] = E.float_to_bf16(-96.0)
    w = rng.uniform(0, 1, rows).astype(np.float32)
    w[3] = 0.0
    w[4] = 1e-20
    codes, scales, cnt = oracle.swiglu_cast(x, w, group, clamp, fmt, sfmt)
    y, cnt_y = oracle.swiglu_forward(x, w, clamp)
    total = 0
    for r in range(rows):
        gate, up = x[r, :hidden].tolist(), x[r, hidden:].tolist()
        ey, ec = E.swiglu_row(gate, up, float(w[r]), clamp)
        total += ec
        assert [float(v) for v in y[r]] == ey
        assert np.array_equal(np.signbit(y[r]), np.signbit(np.array(ey, dtype=np.float32)))
        ecodes, escales = E.cast_row(ey, group, fmt, sfmt)
        if fmt == 4:
            ecodes = E.pack_fp4(ecodes)
        assert codes[r].tolist() == ecodes, r
        assert scales[r].tolist() == escales, r
    assert cnt == total == cnt_y


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_fused_equals_composition(name):
    w = wl.WORKLOADS[name]
    rows = 24
    x = wl.make_x(w, 1, rows=range(rows))
    wt = wl.make_w(w, 1)[:rows] if wl.num_rows(w, 1) >= rows else np.resize(wl.make_w(w, 1), rows)
    fmt = 8 if w.fmt == "fp8" else 4
    sfmt = 0 if w.scale_fmt == "fp32" else 1
    codes, scales, cnt = oracle.swiglu_cast(x, wt, w.group_size, w.clamp_limit, fmt, sfmt)
    y, cnt_y = oracle.swiglu_forward(x, wt, w.clamp_limit)
    c2, s2 = oracle.cast(y, w.group_size, fmt, sfmt)
    assert np.array_equal(codes, c2) and np.array_equal(scales.view(np.uint8), s2.view(np.uint8))
    assert cnt == cnt_y
    # batch invariance: a slice computed alone equals the same rows of the batch
    c3, s3, _ = oracle.swiglu_cast(x[5:11], wt[5:11], w.group_size, w.clamp_limit, fmt, sfmt)
    assert np.array_equal(c3, codes[5:11]) and np.array_equal(s3.view(np.uint8), scales[5:11].view(np.uint8))


def _spacing(v: Fr, fmt: int) -> Fr:
    a = abs(v)
    if fmt == 8:
        if a < Fr(2) ** -6:
            return Fr(2) ** -9
        e = math.floor(math.log2(a))
        return Fr(2) ** (e - 3)
    if a < 1:
        return Fr(1, 2)
    e = math.floor(math.log2(a))
    return Fr(2) ** (e - 1)


@pytest.mark.parametrize("fmt,sfmt,group", [(8, 0, 0), (8, 1, 128), (4, 1, 32), (4, 0, 0), (8, 0, 128)])
def test_invariants(fmt, sfmt, group):
    w_ = wl.WORKLOADS["fp8_g128_ue8m0_n32768_h2048"]
    rows, hidden = 6, w_.hidden
    x = wl.make_x(w_, 2, rows=range(rows))
    wt = wl.make_w(w_, 2)[:rows].copy()
    wt[0] = 0.0
    codes, scales, _ = oracle.swiglu_cast(x, wt, group, None, fmt, sfmt)
    y, _ = oracle.swiglu_forward(x, wt, None)
    fmt_max = 448.0 if fmt == 8 else 6.0
    G = group or hidden
    # zero routing weight: every code is a zero of the value's sign
    if fmt == 8:
        assert set(codes[0].tolist()) <= {0x00, 0x80}
        per_elem = codes
    else:
        assert set((codes[0] & 0x7).tolist()) == {0}
        per_elem = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(rows, hidden)
    assert (scales[0] == 0).all() if sfmt == 0 else (scales[0] == 0).all()
    for r in range(1, rows):
        for k in range(hidden // G):
            grp = y[r, k * G:(k + 1) * G]
            amax = float(np.abs(grp).max())
            if sfmt == 0:
                s = float(scales[r, k])
                assert s == E.round_f32(Fr(amax) / Fr(fmt_max))  # scale = RN(amax / fmt_max)
                s_fr = Fr(s)
            else:
                kk = int(scales[r, k]) - 127
                assert Fr(fmt_max) * Fr(2) ** kk >= Fr(amax) > Fr(fmt_max) * Fr(2) ** (kk - 1)  # minimal
                s_fr = Fr(2) ** kk
            for j in range(0, G, 7):  # dequantisation error within half a step (+ fp32 slack)
                v = E.decode(int(per_elem[r, k * G + j]), fmt)
                yv = Fr(float(grp[j]))
                assert abs(v * s_fr - yv) <= _spacing(v, fmt) * s_fr / 2 + abs(yv) * Fr(1, 2 ** 21)


def test_clamp_count_and_infinite_limit():
    w_ = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    rows = 16
    x = wl.make_x(w_, 0, rows=range(rows))
    wt = wl.make_w(w_, 0)[:rows]
    _, cnt = oracle.swiglu_forward(x, wt, 10.0)
    gate = x[:, : w_.hidden].astype(np.uint32) << 16
    assert cnt == int((gate.view(np.float32) > 10.0).sum()) > 0
    a = oracle.swiglu_cast(x, wt, 0, math.inf, 8, 0)
    b = oracle.swiglu_cast(x, wt, 0, None, 8, 0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2] == 0


def test_scale_layouts_match_hand_written_fixture():
    d = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "scale_layouts.json")))
    s8 = np.array([[10 * r + k for k in range(6)] for r in range(5)], dtype=np.uint8)
    cm = oracle.scale_layout(s8, "ue8m0_colmajor", 255)
    assert len(cm) == 6 * d["ue8m0_colmajor_ld"]
    assert cm[:32].tolist() == d["ue8m0_colmajor_first_two_columns"]
    pk = oracle.scale_layout(s8, "ue8m0_packed", 255).view("<u4")
    assert [f"{w:08x}" for w in pk] == d["ue8m0_packed_words_hex"]
    sf = np.array([[r + k / 8 for k in range(6)] for r in range(5)], dtype=np.float32)
    fc = oracle.scale_layout(sf, "fp32_colmajor", 0).view(np.float32).reshape(6, d["fp32_colmajor_ld"])
    assert fc[1, :5].tolist() == d["fp32_colmajor_column_1"]


# ---------------------------------------------------------------------------
# Top-k gating: the oracle's iterative selection against brute force by sorting
# ---------------------------------------------------------------------------
def _brute_topk(s, k, n_group, topk_group, normalise):
    E = len(s)
    per = E // n_group
    allowed = set(range(E))
    if n_group > 1:
        gsum = []
        for g in range(n_group):
            vals = sorted((float(v) for v in s[g * per:(g + 1) * per]), reverse=True)
            v = float(np.float32(vals[0]) + np.float32(vals[1]))
            gsum.append(-math.inf if math.isnan(v) else v)  # +inf + -inf ranks as -inf
        groups = sorted(range(n_group), key=lambda g: (-gsum[g], g))[:topk_group]
        allowed = {e for g in groups for e in range(g * per, (g + 1) * per)}
    order = sorted(allowed, key=lambda e: (-float(s[e]), e))[:k]
    w = [np.float32(s[e]) for e in order]
    if normalise:
        tot = np.float32(0)
        for v in w:
            tot = np.float32(tot + v)
        if tot != 0:
            w = [np.float32(v / tot) for v in w]
    return order, [float(v) for v in w]


@pytest.mark.parametrize("E,k,ng,tg", [(256, 8, 8, 4), (256, 8, 1, 1), (64, 6, 1, 1), (128, 4, 4, 2), (8, 2, 1, 1),
                                       (72, 5, 3, 2), (256, 256, 1, 1), (32, 1, 16, 3)])
@pytest.mark.parametrize("normalise", [False, True])
def test_topk_gate_matches_brute_force(E, k, ng, tg, normalise):
    rng = np.random.default_rng(E * 7 + k)
    T = 40
    s = np.floor(rng.uniform(0, 1, (T, E)) * 16) / 16  # coarse values: many ties
    s[::5] = rng.uniform(0, 1, (len(s[::5]), E))
    s[3, :] = 0.25
    s[4, ::2] = -0.0
    s[4, 1::2] = 0.0
    s = s.astype(np.float32)
    idx, w = oracle.topk_gate(s, k, ng, tg, normalise)
    for t in range(T):
        order, ww = _brute_topk(s[t], k, ng, tg, normalise)
        assert idx[t].tolist() == order, t
        assert w[t].tolist() == ww, t


@pytest.mark.parametrize("ng,tg", [(8, 4), (8, 7), (4, 2), (16, 3)])
def test_topk_gate_infinite_scores_and_nan_group_sums(ng, tg):
    """Groups whose two best scores are +inf and -inf (a NaN sum, ranked as
    -inf) at every group position, whole groups of -inf, +inf pairs and
    finite rows, against brute force by sorting."""
    E, k = 256, 8
    per = E // ng
    rng = np.random.default_rng(ng * 31 + tg)
    T = 3 * ng + 6
    s = rng.uniform(-1, 1, (T, E)).astype(np.float32)
    for t in range(T):
        g = t % ng
        if t < 2 * ng:  # group g: one +inf, the rest -inf (NaN sum)
            s[t, g * per:(g + 1) * per] = -np.inf
            s[t, g * per + (t % per)] = np.inf
        if ng <= t < 2 * ng:  # and the next group all -inf (a -inf sum that ties with it)
            h = (g + 1) % ng
            s[t, h * per:(h + 1) * per] = -np.inf
        elif 2 * ng <= t < 3 * ng:  # two +inf in group g (an +inf sum)
            s[t, g * per] = s[t, g * per + 1] = np.inf
    kk = min(k, tg * per)
    idx, w = oracle.topk_gate(s, kk, ng, tg, False)
    for t in range(T):
        order, ww = _brute_topk(s[t], kk, ng, tg, False)
        assert idx[t].tolist() == order, (t, idx[t].tolist(), order)
        assert w[t].tolist() == ww, t
    # the NaN group of the first rows is never kept while tg finite groups remain
    for t in range(ng):
        if tg < ng:
            assert not any(int(e) // per == t % ng for e in idx[t]), t


def test_topk_gate_invariants():
    rng = np.random.default_rng(1)
    s = rng.uniform(-1, 1, (30, 256)).astype(np.float32)
    idx, w = oracle.topk_gate(s, 8, 8, 4, False)
    for t in range(30):
        assert len(set(idx[t].tolist())) == 8                  # distinct experts
        assert (np.diff(w[t]) <= 0).all()                     # best first
        groups = {int(e) // 32 for e in idx[t]}
        assert len(groups) <= 4                               # only the kept groups
    idx1, _ = oracle.topk_gate(s, 1, 1, 1, False)
    assert (idx1[:, 0] == np.argmax(s, axis=1)).all()         # k = 1: argmax, first index on ties
    _, wn = oracle.topk_gate(np.abs(s), 8, 8, 4, True)
    assert np.allclose(wn.sum(axis=1), 1.0, atol=1e-6)


def test_scale_inverse_is_rn_of_fmt_max_over_amax():
    """Reading r6: codes come from q = RN(y * RN(fmt_max/amax)), not from the
    reciprocal of the rounded scale.  For amax = 0x1.852eb2p+6 the two
    inverses differ by one ulp, and y = 0x1.d89422p-3 makes
    RN(y * RN(448/amax)) exactly 1.0625, the E4M3 midpoint between 1.0 (0x38)
    and 1.125 (0x39), which goes to the even code 0x38; the other inverse
    lands one ulp above the midpoint and would give 0x39."""
    amax = float.fromhex("0x1.852eb2p+6")
    y = float.fromhex("0x1.d89422p-3")
    inv = E.div_f32(448.0, amax)
    assert E.mul_f32(y, inv) == 1.0625
    assert E.mul_f32(y, E.div_f32(1.0, E.div_f32(amax, 448.0))) > 1.0625
    row = np.zeros((1, 16), dtype=np.float32)
    row[0, 0], row[0, 1], row[0, 2] = amax, y, -y
    codes, scales = oracle.cast(row, 0, 8, 0)
    want_codes, want_scales = E.cast_row([float(v) for v in row[0]], 0, 8, 0)
    assert codes[0].tolist() == want_codes
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x38 and codes[0, 2] == 0xB8
    assert scales[0, 0] == np.float32(want_scales[0])


# ---------------------------------------------------------------------------
# The stand-alone cast of bf16 rows against the exact evaluator
# ---------------------------------------------------------------------------
def _bf16_cast_rows():
    """Four bf16 rows of 16 values, built so that each row's abs-max makes the
    codes land on known ties: row 0 has amax 448 (fp32 inverse exactly 1, so
    1.0625 and 1.1875 are E4M3 midpoints, and 6's inverse makes 0.25 .. 5 E2M1
    midpoints in the FP4 groups), row 1 signed zeros and the smallest bf16
    subnormals, row 2 values whose last mantissa bit is set (a widening that
    dropped it would move them), row 3 an all-zero group next to a huge one."""
    f = E.float_to_bf16
    odd = lambda v: E.bf16_to_float((E.float_to_bf16(v) | 1))  # noqa: E731  last mantissa bit set
    rows = [
        [448.0, 1.0625, -1.1875, 0.25, 0.75, -1.25, 2.5, 5.0, 6.0, 0.25, -0.75, 1.75, 3.5, -5.0, 1.25, 2.5],
        [-0.0, 0.0, 2.0 ** -133, -(2.0 ** -133), 2.0 ** -127, 3 * 2.0 ** -130, -0.0, 0.0,
         1.5 * 2.0 ** -127, -(1.25 * 2.0 ** -127), 2.0 ** -126, -(2.0 ** -126), -0.0, 2.0 ** -133, 0.0,
         -(2.0 ** -132)],
        [odd(1.0), -odd(1.0), odd(3.0), odd(255.0), -odd(250.0), odd(0.5), 127.5, -63.75,
         odd(1.5), odd(2.0), -odd(4.0), odd(8.0), odd(16.0), -odd(32.0), odd(64.0), -odd(128.0)],
        [0.0, -0.0, 0.0, 0.0, -0.0, 0.0, 0.0, -0.0, 1.5 * 2.0 ** 127, -(1.25 * 2.0 ** 126), 2.0 ** 100, 1.0, -1.0,
         0.5, 7.0, -2.0 ** 127],
    ]
    return np.array([[f(v) for v in r] for r in rows], dtype=np.uint16)


@pytest.mark.parametrize("group,fmt,sfmt", [(0, 8, 0), (0, 8, 1), (8, 8, 0), (8, 8, 1), (0, 4, 0), (0, 4, 1),
                                            (8, 4, 1), (8, 4, 0), (4, 4, 1), (2, 8, 0)], ids=str)
def test_cast_bf16_matches_exact_evaluator(group, fmt, sfmt):
    """oracle_cast_bf16 on several rows (a row-stride mistake reads the wrong
    row), groups (a scale-index mistake writes the wrong scale) and ties,
    signed zeros and subnormals (a widening mistake changes a code): every
    code and scale against the exact-rational evaluator on the bf16 values
    widened by hand."""
    x = _bf16_cast_rows()
    codes, scales = oracle.cast_bf16(x, group, fmt, sfmt)
    for r in range(x.shape[0]):
        vals = [E.bf16_to_float(int(h)) for h in x[r]]
        ecodes, escales = E.cast_row(vals, group, fmt, sfmt)
        if fmt == 4:
            ecodes = E.pack_fp4(ecodes)
        assert codes[r].tolist() == ecodes, r
        got = [float(v) for v in scales[r]] if sfmt == 0 else scales[r].tolist()
        assert got == escales, r


def test_cast_bf16_hand_ties():
    """Hand-read codes of row 0 per-token with an fp32 scale: amax 448 gives
    scale 1 and inverse 1, so the codes are the plain E4M3 casts: 448 -> 0x7E,
    1.0625 (midway between 1 = 0x38 and 1.125 = 0x39) -> 0x38, -1.1875 (midway
    between 1.125 and 1.25 = 0x3A) -> 0xBA, 0.25 = 2^-2 -> 0x28, 0.75 = 1.5 * 2^-1 -> 0x34."""
    codes, scales = oracle.cast_bf16(_bf16_cast_rows()[:1], 0, 8, 0)
    assert scales[0, 0] == 1.0
    assert codes[0, :5].tolist() == [0x7E, 0x38, 0xBA, 0x28, 0x34]


# ---------------------------------------------------------------------------
# Rows that pin the fused form's scale step on its own
# ---------------------------------------------------------------------------
def test_fused_scale_inverse_is_rn_of_fmt_max_over_amax():
    """Reading r6 on the fused form.  Gate 0x400b (2.171875) with up 0x3f86
    (1.046875) gives the row's abs-max y0 = 0x1.0541e4p+1; gate 0x400b with up
    0x3dc9 (0.0981...) gives y1 = 0x1.87e2d6p-3 (no weight).  With
    inv = RN(448 / y0), RN(y1 * inv) lands in E4M3 code 0x62; the reciprocal
    of the rounded scale, RN(1 / RN(y0 / 448)), is one ulp larger and moves it
    to 0x63.  The row was found by a search over bf16 pairs whose two inverses
    differ; every value here is re-derived by the exact evaluator."""
    gate = [0x400B, 0x400B] + [0] * 6
    up = [0x3F86, 0x3DC9] + [0] * 6
    x = np.array([gate + up], dtype=np.uint16)
    codes, scales, _ = oracle.swiglu_cast(x, None, 0, None, 8, 0)
    y, _ = E.swiglu_row(gate, up, None, None)
    assert y[0] == float.fromhex("0x1.0541e4p+1") and y[1] == float.fromhex("0x1.87e2d6p-3")
    want_codes, want_scales = E.cast_row(y, 0, 8, 0)
    assert codes[0].tolist() == want_codes and want_codes[:2] == [0x7E, 0x62]
    assert float(scales[0, 0]) == want_scales[0]
    alt_inv = E.div_f32(1.0, E.div_f32(y[0], 448.0))
    assert alt_inv != E.div_f32(448.0, y[0])
    assert E.nearest_code(E.mul_f32(y[1], alt_inv), E.E4M3, 0x80) == 0x63


@pytest.mark.parametrize("fmt,gate,up,byte", [
    (8, 28.0, 16.0, 127),      # sigma(28) = 1 in fp32: amax = 448 exactly, k = 0
    (8, 28.0, 32.0, 128),      # amax = 896 = 448 * 2, k = 1
    (8, 24.0, 0.4375, 122),    # amax = 10.5 = 448 * 2^-5.4..: k = -5 (448/32 = 14 >= 10.5 > 7)
    (4, 24.0, 0.25, 127),      # amax = 6 exactly
    (4, 24.0, 0.125, 126),     # amax = 3 = 6 / 2
    (4, 20.0, 0.5, 128),       # amax = 10: 6 < 10 <= 12
], ids=str)
def test_fused_ue8m0_amax_on_and_near_a_power_of_two_boundary(fmt, gate, up, byte):
    """UE8M0 on the fused form when the group's abs-max equals fmt_max * 2^k
    exactly (the smallest k then satisfies fmt_max * 2^k = amax, so k, not
    k + 1) and when it lies between two such values.  The gates are large
    enough that sigma rounds to 1 in fp32, so amax = gate * up exactly."""
    f = E.float_to_bf16
    g = [f(gate), f(gate / 2), 0, 0, f(-1.0), 0, 0, 0]
    u = [f(up), f(up), 0, 0, f(up), 0, 0, 0]
    x = np.array([g + u, g[::-1] + u[::-1]], dtype=np.uint16)
    codes, scales, _ = oracle.swiglu_cast(x, None, 0, None, fmt, 1)
    for r in range(2):
        y, _ = E.swiglu_row(x[r, :8].tolist(), x[r, 8:].tolist(), None, None)
        ecodes, escales = E.cast_row(y, 0, fmt, 1)
        if fmt == 4:
            ecodes = E.pack_fp4(ecodes)
        assert escales == [byte]
        assert scales[r].tolist() == [byte] and codes[r].tolist() == ecodes
