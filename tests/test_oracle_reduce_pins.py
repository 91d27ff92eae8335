"""Pins of the oracle's weighted top-k reduce ("【DeepSeek】TileKernels从入门到精通"
ch.3 "结算中心的“减法工程”" and "动态寻址") against things other than itself:
torch's fp32 -> bf16 conversion, exact integer arithmetic, an exact-rational
evaluator (tests/exact.py), an error bound, and invariants of the definition.
"""
import struct

import numpy as np
import pytest
import torch

import exact as E
import oracle
from moe_activation_bit_amd import workloads as wl


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bits of fp32 values that are exactly bf16."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32)
    assert (b & 0xFFFF == 0).all()
    return (b >> 16).astype(np.uint16)


def bf16_value(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


def test_bf16_output_rounding_matches_torch():
    """k = 1, x = 1, no row scale, global scale 1: the fp32 result is the
    weight itself, so the bf16 output is the weight rounded to bf16.  Swept
    over ties, subnormals, values near the top of the range and random bit
    patterns, against torch's fp32 -> bf16 conversion."""
    rng = np.random.default_rng(11)
    special = []
    for hi in (0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x4049, 0x7F7E, 0x7F7F):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            special.append((hi << 16) | lo)
    bits = np.concatenate([np.array(special, dtype=np.uint32),
                           rng.integers(0, 0x7F800000, 20000, dtype=np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000])
    w = bits.view(np.float32).reshape(-1, 1)
    x = bf16_bits(np.ones((1, 8), dtype=np.float32))
    pos = np.zeros((len(w), 1), dtype=np.int32)
    # the sum starts from +0, so a -0 weight gives +0 (+0 + -0 = +0)
    expect = np.repeat(np.where(w == 0, np.float32(0.0), w), 8, axis=1)
    got = oracle.moe_reduce(x, pos, w, None, 1.0, out_bf16=True)
    want = torch.from_numpy(expect).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    f32 = oracle.moe_reduce(x, pos, w, None, 1.0, out_bf16=False)
    assert np.array_equal(f32.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("k,drop,with_scale", [(1, 0.0, False), (2, 0.0, True), (8, 0.2, True), (6, 0.5, False),
                                               (16, 0.1, True)])
def test_exact_integer_case(k, drop, with_scale):
    """Small integers times powers of two: every product and sum is exact in
    fp32, so the oracle must equal the float64 gather-weight-sum written with
    numpy fancy indexing (checks pos, the slot order of w, the row of each
    scale, dropped slots and out-of-range rows)."""
    rng = np.random.default_rng(k * 100 + int(drop * 10))
    tokens, hidden, n_rows = 37, 24, 150
    xv = rng.integers(-64, 65, (n_rows, hidden)).astype(np.float32)
    x = bf16_bits(xv)
    pos = rng.integers(0, n_rows, (tokens, k)).astype(np.int32)
    d = rng.random((tokens, k)) < drop
    pos[d] = np.where(rng.random(d.sum()) < 0.5, -1, n_rows + rng.integers(0, 5, d.sum()))
    w = (2.0 ** -rng.integers(0, 4, (tokens, k))).astype(np.float32) * rng.choice([-1, 1], (tokens, k))
    rs = (2.0 ** rng.integers(-2, 3, n_rows)).astype(np.float32) if with_scale else None
    gs = 2.0
    present = (pos >= 0) & (pos < n_rows)
    safe = np.where(present, pos, 0)
    scale = rs[safe] if with_scale else np.ones_like(w)
    want = gs * np.einsum("tk,tkh->th", np.where(present, w * scale, 0.0).astype(np.float64),
                          xv[safe].astype(np.float64))
    got32 = oracle.moe_reduce(x, pos, w, rs, gs, out_bf16=False)
    assert np.array_equal(got32.astype(np.float64), want)
    got16 = oracle.moe_reduce(x, pos, w, rs, gs, out_bf16=True)
    assert np.array_equal(got16, torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))


def test_matches_exact_evaluator_on_random_floats():
    """Random bf16 rows, weights and scales: every element of the fp32 and bf16
    outputs against the exact-rational evaluation of the stated rounding
    sequence."""
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, w, rs, n_rows = wl.make_routing(r, 4)
    pos, w = pos[:6], w[:6]
    rows = sorted(set(int(p) for p in pos.ravel() if p >= 0))
    xfull = np.zeros((n_rows, 16), dtype=np.uint16)
    xfull[rows] = wl.make_expert_rows(r, 4, n_rows, rows)[:, :16]
    got32 = oracle.moe_reduce(xfull, pos, w, rs, r.global_scale, out_bf16=False)
    got16 = oracle.moe_reduce(xfull, pos, w, rs, r.global_scale, out_bf16=True)
    for t in range(pos.shape[0]):
        slots = [j for j in range(pos.shape[1]) if pos[t, j] >= 0]
        for c in range(16):
            v = E.reduce_cell([int(xfull[pos[t, j], c]) for j in slots], [float(w[t, j]) for j in slots],
                              [float(rs[pos[t, j]]) for j in slots], r.global_scale)
            assert struct.pack("<f", v) == struct.pack("<f", float(got32[t, c])), (t, c)
            assert E.round_bf16(v) == int(got16[t, c]), (t, c)


def test_slot_order_is_the_accumulation_order():
    """Terms 1, 2^-24, 2^-24 summed in slot order stay 1 (each addition is a
    tie that rounds back to 1); summed smallest first they give 1 + 2^-23."""
    x = bf16_bits(np.array([[1.0] * 8, [2.0 ** -24] * 8], dtype=np.float32))
    w = np.ones((1, 3), dtype=np.float32)
    fwd = oracle.moe_reduce(x, np.array([[0, 1, 1]], dtype=np.int32), w, out_bf16=False)
    rev = oracle.moe_reduce(x, np.array([[1, 1, 0]], dtype=np.int32), w, out_bf16=False)
    assert (fwd == 1.0).all()
    assert (rev == np.float32(1.0 + 2.0 ** -23)).all()


def test_error_bound_against_float64():
    """On the small workload the fp32 result is within the textbook bound of
    recursive summation: |out - exact| <= (k+2) u sum|terms| |g| (u = 2^-24)."""
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, w, rs, n_rows = wl.make_routing(r, 1)
    x = wl.make_expert_rows(r, 1, n_rows)
    got = oracle.moe_reduce(x, pos, w, rs, r.global_scale, out_bf16=False).astype(np.float64)
    xv = bf16_value(x).astype(np.float64)
    present = pos >= 0
    safe = np.where(present, pos, 0)
    f = np.where(present, w.astype(np.float64) * rs[safe], 0.0)
    terms = f[:, :, None] * xv[safe]
    exact = terms.sum(axis=1) * r.global_scale
    bound = (r.k + 2) * 2.0 ** -24 * np.abs(terms).sum(axis=1) * abs(r.global_scale) + 1e-30
    assert (np.abs(got - exact) <= bound).all()
    assert np.abs(got - exact).max() > 0  # rounding does happen


def test_invariants():
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, w, rs, n_rows = wl.make_routing(r, 2)
    x = wl.make_expert_rows(r, 2, n_rows)[:, :40].copy()
    base = oracle.moe_reduce(x, pos, w, rs, r.global_scale)
    # relabelling the rows (permuting x and the scales with the map) changes nothing
    perm = np.random.default_rng(3).permutation(n_rows)
    inv = np.argsort(perm)
    pos2 = np.where(pos >= 0, inv[np.maximum(pos, 0)], -1).astype(np.int32)
    assert np.array_equal(oracle.moe_reduce(x[perm], pos2, w, rs[perm], r.global_scale), base)
    # a dropped slot is the same as an out-of-range row ...
    pos3 = np.where(pos >= 0, pos, n_rows + 7).astype(np.int32)
    assert np.array_equal(oracle.moe_reduce(x, pos3, w, rs, r.global_scale), base)
    # ... and as no slot at all: a token's present slots moved to the front
    # (order kept), the rest dropped
    for t in range(pos.shape[0]):
        keep = pos[t] >= 0
        pc = np.full((1, pos.shape[1]), -1, dtype=np.int32)
        wc = np.zeros((1, pos.shape[1]), dtype=np.float32)
        pc[0, :keep.sum()], wc[0, :keep.sum()] = pos[t][keep], w[t][keep]
        assert np.array_equal(oracle.moe_reduce(x, pc, wc, rs, r.global_scale)[0], base[t])
    # a token with every slot dropped gives signed zeros: +0, or -0 for a negative global scale
    pos4 = pos.copy()
    pos4[5] = -1
    out = oracle.moe_reduce(x, pos4, w, rs, -1.0)
    assert (out[5] == 0x8000).all()
    assert (oracle.moe_reduce(x, pos4, w, rs, 1.0)[5] == 0).all()
    # tokens are independent: a subset of tokens gives the same rows
    assert np.array_equal(oracle.moe_reduce(x, pos[10:20], w[10:20], rs, r.global_scale), base[10:20])
    # the map is range-checked, not trusted: n_rows = 0 drops everything
    assert (oracle.moe_reduce(x[:0], pos, w, None, 1.0) == 0).all()


def test_routing_generator_structure():
    """The input recipe: each present (token, slot) owns one row, rows are
    grouped by expert with tokens in order inside an expert, weights sum to 1."""
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, w, rs, n_rows = wl.make_routing(r, 0)
    p = pos[pos >= 0]
    assert np.array_equal(np.sort(p), np.arange(n_rows))
    assert 0 < (pos < 0).sum() < pos.size * 0.15
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert rs.shape == (n_rows,) and (rs >= 0.5).all() and (rs < 2.0).all()
    # within one token's slots the rows are distinct
    for t in range(pos.shape[0]):
        q = pos[t][pos[t] >= 0]
        assert len(set(q.tolist())) == len(q)


# ---- the token/top-k -> position map ("动态寻址")

def test_topk_to_pos_hand_cases():
    """Hand-worked cases (tests/golden/topk_to_pos.json): repeated, negative
    and out-of-range experts, an expert nobody picks, slot order unlike expert
    order, one expert, no present slot."""
    import json
    import os
    d = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "topk_to_pos.json")))
    for c in d["cases"]:
        pos, off = oracle.topk_to_pos(np.array(c["idx"], dtype=np.int32), c["experts"])
        assert pos.tolist() == c["pos"], c["name"]
        assert off.tolist() == c["offsets"], c["name"]


def _pos_by_sorting(idx: np.ndarray, experts: int):
    """The same map by a different route: list the present slots as (expert,
    token, slot), sort them, and number them in that order."""
    tokens, k = idx.shape
    present = []
    for t in range(tokens):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < experts and e not in seen:
                present.append((e, t, j))
            seen.add(e)
    pos = np.full((tokens, k), -1, dtype=np.int64)
    for row, (e, t, j) in enumerate(sorted(present)):
        pos[t, j] = row
    experts_of_rows = np.array([e for e, _, _ in sorted(present)], dtype=np.int64)
    off = np.searchsorted(experts_of_rows, np.arange(experts + 1), side="left")
    return pos, off


@pytest.mark.parametrize("seed", range(12))
def test_topk_to_pos_matches_a_stable_sort(seed):
    rng = np.random.default_rng(seed)
    tokens, k, experts = int(rng.integers(0, 40)), int(rng.integers(1, 6)), int(rng.integers(1, 9))
    idx = rng.integers(-2, experts + 2, size=(tokens, k)).astype(np.int32)  # repeats, -1/-2, past the end
    pos, off = oracle.topk_to_pos(idx, experts)
    want_pos, want_off = _pos_by_sorting(idx, experts)
    assert np.array_equal(pos, want_pos)
    assert np.array_equal(off, want_off)


def test_topk_to_pos_invariants():
    """On a top-k shaped routing (distinct experts per token, a few dropped
    slots): the present slots take every row in [0, total) once, expert e's
    rows are [offsets[e], offsets[e+1]) and hold its tokens in increasing
    order, and absent slots are -1."""
    rng = np.random.default_rng(5)
    tokens, k, experts = 3000, 8, 256
    idx = np.stack([rng.choice(experts, size=k, replace=False) for _ in range(tokens)]).astype(np.int32)
    idx[rng.random((tokens, k)) < 0.05] = -1
    pos, off = oracle.topk_to_pos(idx, experts)
    present = idx >= 0
    assert (pos[~present] == -1).all()
    total = int(present.sum())
    assert off[0] == 0 and off[-1] == total and (np.diff(off) >= 0).all()
    assert np.array_equal(np.sort(pos[present]), np.arange(total))
    for e in range(experts):
        t_of = np.nonzero((idx == e).any(axis=1))[0]
        rows = pos[idx == e]
        assert np.array_equal(rows, np.arange(off[e], off[e + 1]))
        assert len(t_of) == off[e + 1] - off[e]
