"""GPU parity of the weighted top-k reduce (tk_moe_reduce) against the oracle,
bit-exact: the small and the full-size workload on every element, every k
the kernel specialises for, ragged and tiny hidden sizes, dropped and
out-of-range slots, repeated rows, the bf16 rounding of the output, and the
degenerate cases (no tokens, no rows, every slot dropped)."""
import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
import oracle
from moe_activation_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
OK = tk.TkStatus.TK_OK
PAD = 256


def say(*a):
    print("[gpu-case]", *a, flush=True)


def run_reduce(x, pos, w, rs, gs, out_bf16, n_rows=None):
    """Call tk_moe_reduce on device copies; check the canaries around the
    output and return it as numpy (bf16 bits uint16, or fp32)."""
    tokens, k = pos.shape
    hidden = x.shape[1]
    n_rows = x.shape[0] if n_rows is None else n_rows
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV) if x.size else None
    pd = torch.from_numpy(np.ascontiguousarray(pos)).to(DEV)
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(DEV)
    rd = torch.from_numpy(np.ascontiguousarray(rs)).to(DEV) if rs is not None else None
    item = 2 if out_bf16 else 4
    obuf = torch.full((tokens * hidden * item + 2 * PAD,), 0xC3, dtype=torch.uint8, device=DEV)
    rc = tk.tk_moe_reduce(xd, rd, pd, wd, gs, tokens, k, hidden, n_rows,
                          tk.TK_DTYPE_BF16 if out_bf16 else tk.TK_DTYPE_FP32, obuf.data_ptr() + PAD)
    assert rc == OK, tk.tk_status_str(rc)
    torch.cuda.synchronize()
    o = obuf.cpu().numpy()
    assert (o[:PAD] == 0xC3).all() and (o[len(o) - PAD:] == 0xC3).all(), "output canary overwritten"
    body = o[PAD:len(o) - PAD]
    return (body.view(np.uint16) if out_bf16 else body.view(np.float32)).reshape(tokens, hidden)


def same(got, want, what):
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        t, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} elements differ, first token {t} col {c}: "
                             f"{got[t, c]:#x} vs {want[t, c]:#x}")


@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("with_scale", [True, False])
def test_small_workload_matches_oracle(out_bf16, with_scale):
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    say("reduce small", out_bf16, with_scale)
    pos, w, rs, n_rows = wl.make_routing(r, 0)
    x = wl.make_expert_rows(r, 0, n_rows)
    rs = rs if with_scale else None
    got = run_reduce(x, pos, w, rs, r.global_scale, out_bf16)
    same(got, oracle.moe_reduce(x, pos, w, rs, r.global_scale, out_bf16), "small")


def random_case(seed, tokens, k, hidden, n_rows, drop=0.1, bad=0.05):
    """Random map with repeated rows, dropped (-1) and out-of-range entries;
    rows drawn as bf16 N(0, 1) through the workload module's generator."""
    rng = np.random.default_rng(seed)
    r = wl.ReduceWorkload(f"reduce_case_{seed}", tokens, k, 8, hidden, 1.0, 0.0, True, 1.0, True)
    x = wl.make_expert_rows(r, seed, n_rows)
    pos = rng.integers(0, max(n_rows, 1), (tokens, k)).astype(np.int32)
    u = rng.random((tokens, k))
    pos[u < drop] = -1
    pos[(u >= drop) & (u < drop + bad)] = n_rows + rng.integers(0, 1000)
    if tokens > 3:
        pos[3] = -1  # one token with every slot dropped
    w = rng.standard_normal((tokens, k)).astype(np.float32)
    rs = rng.uniform(0.25, 4.0, n_rows).astype(np.float32)
    return x, pos, w, rs


KS = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 24, 32, 33, 40, 48, 63, 64]  # above 32: batches of 32 rows


@pytest.mark.parametrize("k", KS)
def test_every_k(k):
    say("reduce k", k)
    x, pos, w, rs = random_case(100 + k, 45, k, 2048 + 8 * k, 300)
    for out_bf16 in (True, False):
        got = run_reduce(x, pos, w, rs, -1.75, out_bf16)
        same(got, oracle.moe_reduce(x, pos, w, rs, -1.75, out_bf16), f"k={k} bf16={out_bf16}")


HIDDENS = [8, 56, 512, 520, 1000, 1024, 1536, 3584, 4104, 7168, 7176]


@pytest.mark.parametrize("hidden", HIDDENS)
def test_hidden_sizes_and_ragged_tails(hidden):
    say("reduce hidden", hidden)
    for k in (2, 8):
        x, pos, w, rs = random_case(hidden + k, 33, k, hidden, 120)
        got = run_reduce(x, pos, w, rs, 2.5, True)
        same(got, oracle.moe_reduce(x, pos, w, rs, 2.5, True), f"hidden={hidden} k={k}")
        got = run_reduce(x, pos, w, None, 0.5, False)
        same(got, oracle.moe_reduce(x, pos, w, None, 0.5, False), f"hidden={hidden} k={k} fp32 no-scale")


def test_bf16_rounding_sweep():
    """k = 1, x = 1, no scale: the output is each weight rounded to bf16 by the
    kernel's converter -- ties, subnormals, near-overflow, random patterns."""
    rng = np.random.default_rng(5)
    special = [(hi << 16) | lo for hi in (0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F)
               for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF)]
    bits = np.concatenate([np.array(special, dtype=np.uint32), rng.integers(0, 0x7F800000, 60000, dtype=np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000])
    w = bits.view(np.float32).reshape(-1, 1).copy()
    x = np.full((1, 8), 0x3F80, dtype=np.uint16)
    pos = np.zeros((len(w), 1), dtype=np.int32)
    say("reduce bf16 sweep", len(w))
    got = run_reduce(x, pos, w, None, 1.0, True)
    same(got, oracle.moe_reduce(x, pos, w, None, 1.0, True), "bf16 rounding")


def test_full_size_workload_every_element():
    r = wl.REDUCE_WORKLOADS[wl.REDUCE_HEADLINE]
    say("reduce full size", r.name)
    pos, w, rs, n_rows = wl.make_routing(r, 0)
    x = wl.make_expert_rows(r, 0, n_rows)
    got = run_reduce(x, pos, w, rs, r.global_scale, r.out_bf16)
    same(got, oracle.moe_reduce(x, pos, w, rs, r.global_scale, r.out_bf16), r.name)


def test_degenerate_cases():
    say("reduce degenerate")
    x, pos, w, rs = random_case(7, 16, 8, 1024, 50)
    # every slot dropped: +0 everywhere, -0 for a negative global scale
    allgone = np.full_like(pos, -1)
    assert (run_reduce(x, allgone, w, rs, 3.0, True) == 0).all()
    assert (run_reduce(x, allgone, w, rs, -3.0, True) == 0x8000).all()
    # no rows at all (x may be NULL): every entry is out of range
    got = run_reduce(np.zeros((0, 1024), dtype=np.uint16), pos, w, None, 1.0, False)
    assert (got.view(np.uint32) == 0).all()
    # no tokens: nothing launched, nothing written
    ob = torch.full((64,), 7, dtype=torch.uint8, device=DEV)
    pd = torch.zeros(8, dtype=torch.int32, device=DEV)
    xd = torch.zeros(1024, dtype=torch.int16, device=DEV)
    assert tk.tk_moe_reduce(xd, None, pd, pd, 1.0, 0, 8, 1024, 1, tk.TK_DTYPE_BF16, ob) == OK
    torch.cuda.synchronize()
    assert (ob.cpu().numpy() == 7).all()
    # the same row in every slot of a token
    pos2 = np.repeat(pos[:, :1].clip(0, 49), 8, axis=1)
    got = run_reduce(x, pos2, w, rs, 1.0, True)
    same(got, oracle.moe_reduce(x, pos2, w, rs, 1.0, True), "repeated rows")


def test_bf16_output_reads_as_torch_bf16():
    """The output buffer is ordinary row-major bf16: torch reading it as a
    bfloat16 tensor sees the oracle's values."""
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, w, rs, n_rows = wl.make_routing(r, 3)
    x = wl.make_expert_rows(r, 3, n_rows)
    say("reduce torch view")
    xd = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = torch.empty((r.tokens, r.hidden), dtype=torch.bfloat16, device=DEV)
    rc = tk.tk_moe_reduce(xd, torch.from_numpy(rs).to(DEV), torch.from_numpy(pos).to(DEV),
                          torch.from_numpy(w).to(DEV), r.global_scale, r.tokens, r.k, r.hidden, n_rows,
                          tk.TK_DTYPE_BF16, out)
    assert rc == OK
    want = oracle.moe_reduce(x, pos, w, rs, r.global_scale, True)
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("hidden", [16392, 32768, 65528])
def test_long_rows_and_one_token(hidden):
    """Rows longer than any model's hidden size (ragged and not), and a
    single-token call, against the oracle."""
    say("reduce long rows", hidden)
    x, pos, w, rs = random_case(hidden, 9, 8, hidden, 40)
    got = run_reduce(x, pos, w, rs, 2.5, True)
    same(got, oracle.moe_reduce(x, pos, w, rs, 2.5, True), f"hidden={hidden}")
    got = run_reduce(x, pos[:1], w[:1], rs, 2.5, False)
    same(got, oracle.moe_reduce(x, pos[:1], w[:1], rs, 2.5, False), f"hidden={hidden} one token")
