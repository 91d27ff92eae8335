"""GPU parity of the token/top-k -> expert-row map (tk_topk_to_pos) against the
oracle: every position and offset bit-exact, on top-k shaped routings and on
inputs with dropped, negative, out-of-range and repeated experts, across the
1024-token blocks the kernels split the tokens into."""
import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
import oracle
from moe_activation_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
OK = tk.TkStatus.TK_OK


def routing(tokens, k, experts, seed, drop=0.0, noise=False):
    """A top-k shaped routing (k distinct experts per token); `drop` of the
    slots set to -1; with `noise`, some slots get a repeat of another slot's
    expert, a negative value or one past the last expert."""
    rng = np.random.default_rng(seed)
    if k <= experts:
        idx = np.argsort(rng.random((tokens, experts)), axis=1)[:, :k].astype(np.int32)
    else:
        idx = rng.integers(0, experts, size=(tokens, k)).astype(np.int32)
    idx[rng.random((tokens, k)) < drop] = -1
    if noise and tokens > 0 and k > 1:
        m = rng.random((tokens, k))
        idx[m < 0.03] = experts + rng.integers(0, 3)
        idx[(m >= 0.03) & (m < 0.06)] = -(1 + rng.integers(0, 5))
        rep = (m >= 0.06) & (m < 0.10)
        idx[:, 1:][rep[:, 1:]] = idx[:, :-1][rep[:, 1:]]  # repeat the previous slot's expert
    return idx


def run(idx, experts):
    tokens, k = idx.shape
    d = torch.from_numpy(np.ascontiguousarray(idx)).to(DEV)
    pad = 32
    pos = torch.full((tokens * k + 2 * pad,), 1234567, dtype=torch.int32, device=DEV)
    off = torch.full((experts + 1 + 2 * pad,), 7654321, dtype=torch.int32, device=DEV)
    rc = tk.tk_topk_to_pos(d, tokens, k, experts, pos.data_ptr() + 4 * pad, off.data_ptr() + 4 * pad)
    assert rc == OK, tk.tk_status_str(rc)
    torch.cuda.synchronize()
    p, o = pos.cpu().numpy(), off.cpu().numpy()
    assert (p[:pad] == 1234567).all() and (p[pad + tokens * k:] == 1234567).all(), "pos canary"
    assert (o[:pad] == 7654321).all() and (o[pad + experts + 1:] == 7654321).all(), "offsets canary"
    return p[pad:pad + tokens * k].reshape(tokens, k), o[pad:pad + experts + 1]


CASES = [  # (tokens, k, experts, drop, noise)
    (1, 1, 1, 0.0, False), (3, 2, 3, 0.0, True), (7, 4, 5, 0.2, True), (1023, 8, 256, 0.0, False),
    (1024, 8, 256, 0.0, False), (1025, 8, 256, 0.05, False), (2048, 8, 256, 0.0, True), (4096, 8, 256, 0.0, False),
    (3000, 6, 160, 0.1, True), (2049, 1, 512, 0.0, False), (777, 32, 512, 0.0, True), (777, 32, 64, 0.0, True),
    (5000, 9, 100, 0.0, True), (1500, 2, 2, 0.0, True), (65536, 8, 256, 0.02, False), (40000, 16, 384, 0.0, True),
    # k above 32 (up to 64): one-workgroup calls, blocks of 256 and 1024 tokens, more slots than experts
    (200, 64, 512, 0.0, True), (700, 48, 256, 0.1, True), (200, 64, 32, 0.0, False), (3000, 40, 64, 0.0, True),
    (1100, 64, 512, 0.05, True), (66000, 33, 256, 0.0, False),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_topk_to_pos_matches_oracle(case):
    tokens, k, experts, drop, noise = case
    print("[gpu-case] topk_to_pos", case, flush=True)
    idx = routing(tokens, k, experts, seed=tokens * 31 + k * 7 + experts, drop=drop, noise=noise)
    gp, go = run(idx, experts)
    op, oo = oracle.topk_to_pos(idx, experts)
    assert np.array_equal(go, oo), np.argwhere(go != oo)[:4]
    bad = np.argwhere(gp != op)
    assert bad.size == 0, f"positions differ at {bad[:4].tolist()}"


def test_topk_to_pos_all_slots_absent_and_one_expert():
    """Every slot dropped (all rows of offsets zero, every position -1), and
    one expert named by every token (positions are the token order)."""
    print("[gpu-case] topk_to_pos degenerate", flush=True)
    idx = np.full((3000, 4), -1, dtype=np.int32)
    gp, go = run(idx, 64)
    assert (gp == -1).all() and (go == 0).all()
    idx = np.zeros((2500, 1), dtype=np.int32)
    gp, go = run(idx, 1)
    assert np.array_equal(gp[:, 0], np.arange(2500)) and go.tolist() == [0, 2500]


def test_topk_to_pos_no_tokens_zeroes_the_offsets():
    print("[gpu-case] topk_to_pos no tokens", flush=True)
    off = torch.full((300,), 99, dtype=torch.int32, device=DEV)
    pos = torch.full((4,), 5, dtype=torch.int32, device=DEV)
    idx = torch.zeros((4,), dtype=torch.int32, device=DEV)
    assert tk.tk_topk_to_pos(idx, 0, 8, 256, pos, off) == OK
    torch.cuda.synchronize()
    o = off.cpu().numpy()
    assert (o[:257] == 0).all() and (o[257:] == 99).all() and (pos.cpu().numpy() == 5).all()


@pytest.mark.parametrize("k,ng,tg", [(8, 8, 4), (48, 1, 1), (64, 8, 6)], ids=str)
def test_gating_then_map_then_reduce(k, ng, tg):
    """The gating's indices go straight into the map, and the map into the
    reduce: expert rows laid out by the map and reduced through it give, bit
    for bit, the oracle's reduce over the oracle's map of the oracle's
    gating (k = 8 with groups, and k above 32, which the one-token gating
    kernel, the 64-slot map and the reduce's 32-row batches serve)."""
    print("[gpu-case] gating -> map -> reduce", k, ng, tg, flush=True)
    T, E, hidden = 1500, 256, (1024 if k <= 8 else 256)
    s = wl.uniform(wl.stream_key("pos_test", 0, "scores"), 0, T * E).reshape(T, E).astype(np.float32)
    sd = torch.from_numpy(s).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    assert tk.tk_topk_gate(sd, T, E, k, ng, tg, 1, idx, w) == OK
    pos = torch.empty((T, k), dtype=torch.int32, device=DEV)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    assert tk.tk_topk_to_pos(idx, T, k, E, pos, off) == OK
    torch.cuda.synchronize()
    oi, ow = oracle.topk_gate(s, k, ng, tg, True)
    op, oo = oracle.topk_to_pos(oi, E)
    assert np.array_equal(idx.cpu().numpy(), oi) and np.array_equal(pos.cpu().numpy(), op)
    assert np.array_equal(off.cpu().numpy(), oo)
    n_rows = int(oo[-1])
    rows = (wl.uniform(wl.stream_key("pos_test", 1, "rows"), 0, n_rows * hidden).reshape(n_rows, hidden) * 4 - 2)
    xb = (rows.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation
    out = torch.empty((T, hidden), dtype=torch.bfloat16, device=DEV)
    assert tk.tk_moe_reduce(torch.from_numpy(xb.view(np.int16)).to(DEV), None, pos, w, 1.0, T, k, hidden, n_rows,
                            tk.TK_DTYPE_BF16, out) == OK
    torch.cuda.synchronize()
    want = oracle.moe_reduce(xb, op, ow, None, 1.0, True)
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("tokens", [300, 5000])
def test_topk_to_pos_k8_unaligned(tokens):
    """k = 8 with the index and position arrays 4 bytes past a 16-byte
    boundary: the per-slot loads and stores (16-byte aligned arrays take
    two 16-byte accesses per token) give the same map."""
    print("[gpu-case] topk_to_pos k=8 unaligned", tokens, flush=True)
    E, k = 256, 8
    idx = routing(tokens, k, E, seed=tokens + 77, drop=0.05, noise=True)
    di = torch.zeros(tokens * k + 4, dtype=torch.int32, device=DEV)
    di[1:1 + tokens * k] = torch.from_numpy(idx.reshape(-1)).to(DEV)
    dp = torch.full((tokens * k + 4,), 99, dtype=torch.int32, device=DEV)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    assert (di.data_ptr() + 4) % 16 == 4 and (dp.data_ptr() + 4) % 16 == 4
    assert tk.tk_topk_to_pos(di.data_ptr() + 4, tokens, k, E, dp.data_ptr() + 4, off) == OK
    torch.cuda.synchronize()
    op, oo = oracle.topk_to_pos(idx, E)
    p = dp.cpu().numpy()
    assert p[0] == 99 and (p[1 + tokens * k:] == 99).all()
    assert np.array_equal(p[1:1 + tokens * k].reshape(tokens, k), op)
    assert np.array_equal(off.cpu().numpy(), oo)
