"""The entry points under HIP graph capture: they allocate nothing, record no
memset and query nothing that capture forbids, so a caller can capture them
once and replay.  One graph holds a fused FP8 launch (with the clamp counter),
an FP4 launch, a stand-alone cast, the gating and the position map of its
indices (three launches), the reduce, three launches
of long rows (groups shared by two waves, and 16 streamed steps), segmented
groups of 96 columns (fused and cast) and two-pass groups of 8704 columns;
small launches among them read the 16 KiB table; it is replayed
several times with eager work between the replays (outputs poisoned, the
counter zeroed by torch outside the graph), and every replay must equal the
eager results bit for bit."""
import math

import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
from moe_activation_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
OK = tk.TkStatus.TK_OK


def test_capture_and_replay_matches_eager():
    print("[gpu-case] graph capture", flush=True)
    assert tk.tk_init(0) == OK  # the one-time table set-up happens before capture
    wc = wl.WORKLOADS["fp8_per_token_clamp10_n131072_h2048"]
    n = 512
    x = torch.from_numpy(wl.make_x(wc, 0, rows=range(n)).view(np.int16)).to(DEV)
    w = torch.from_numpy(wl.make_w(wc, 0)[:n]).to(DEV)
    w4 = wl.WORKLOADS["fp4_g32_ue8m0_n65536_h4096"]
    n4 = 256
    x4 = torch.from_numpy(wl.make_x(w4, 0, rows=range(n4)).view(np.int16)).to(DEV)
    r = wl.REDUCE_WORKLOADS["reduce_t64_k8_h7168_drop5"]
    pos, rw, rs, n_rows = wl.make_routing(r, 0)
    xr = torch.from_numpy(wl.make_expert_rows(r, 0, n_rows).view(np.int16)).to(DEV)
    pd, rwd, rsd = torch.from_numpy(pos).to(DEV), torch.from_numpy(rw).to(DEV), torch.from_numpy(rs).to(DEV)
    scores = torch.from_numpy(wl.uniform(wl.stream_key("graph_test", 0, "scores"), 0, 300 * 256)
                              .reshape(300, 256).astype(np.float32)).to(DEV)
    # long rows: per-token groups of 16384 columns (two waves per group, loads
    # streamed) and 8192 columns (one wave, 16 streamed steps)
    nl, hl = 40, 16384
    xl_h = wl.make_x(wc, 1, rows=range(nl))
    xl = torch.from_numpy(np.ascontiguousarray(np.tile(xl_h, (1, 2 * hl // xl_h.shape[1]))).view(np.int16)).to(DEV)

    # segmented groups (96 columns of 2016) and two-pass groups (8704 columns of 17408)
    ns, hs = 300, 2016
    xs = torch.from_numpy(np.ascontiguousarray(np.concatenate(
        [wl.make_x(wc, 2, rows=range(ns))[:, :hs], wl.make_x(wc, 2, rows=range(ns))[:, 2048:2048 + hs]], axis=1))
        .view(np.int16)).to(DEV)
    n2, h2 = 12, 17408
    x2 = torch.from_numpy(np.ascontiguousarray(np.tile(xl_h[:n2], (1, (2 * h2 + 4095) // 4096))[:, :2 * h2])
                          .view(np.int16)).to(DEV)

    outs = dict(
        codes=torch.empty((n, 2048), dtype=torch.uint8, device=DEV),
        scales=torch.empty((n, 1), dtype=torch.float32, device=DEV),
        count=torch.zeros(1, dtype=torch.int64, device=DEV),
        codes4=torch.empty((n4, 2048), dtype=torch.uint8, device=DEV),
        scales4=torch.empty((n4, 128), dtype=torch.uint8, device=DEV),
        ccodes=torch.empty((2 * n, 2048), dtype=torch.uint8, device=DEV),
        cscales=torch.empty((2 * n, 16), dtype=torch.uint8, device=DEV),
        idx=torch.empty((300, 8), dtype=torch.int32, device=DEV),
        gw=torch.empty((300, 8), dtype=torch.float32, device=DEV),
        pos=torch.empty((300, 8), dtype=torch.int32, device=DEV),
        poff=torch.empty((257,), dtype=torch.int32, device=DEV),
        red=torch.empty((r.tokens, r.hidden), dtype=torch.bfloat16, device=DEV),
        lcodes=torch.empty((nl, hl), dtype=torch.uint8, device=DEV),
        lscales=torch.empty((nl, 1), dtype=torch.float32, device=DEV),
        lcodes4=torch.empty((nl, hl // 4), dtype=torch.uint8, device=DEV),
        lscales4=torch.empty((nl, 1), dtype=torch.uint8, device=DEV),
        lccodes=torch.empty((nl, hl), dtype=torch.uint8, device=DEV),
        lcscales=torch.empty((nl, 1), dtype=torch.float32, device=DEV),
        scodes=torch.empty((ns, hs), dtype=torch.uint8, device=DEV),
        sscales=torch.empty((ns, hs // 96), dtype=torch.uint8, device=DEV),
        sccodes=torch.empty((ns, hs), dtype=torch.uint8, device=DEV),
        sccscales=torch.empty((ns, 2 * hs // 96), dtype=torch.float32, device=DEV),
        tcodes=torch.empty((n2, h2), dtype=torch.uint8, device=DEV),
        tscales=torch.empty((n2, 2), dtype=torch.float32, device=DEV),
    )

    def work():
        s = torch.cuda.current_stream()
        assert tk.tk_swiglu_cast_fp8(x, w, n, 2048, 0, 10.0, tk.TK_SCALE_FP32, outs["codes"], outs["scales"],
                                     outs["count"], s) == OK
        assert tk.tk_swiglu_cast_fp4(x4, None, n4, 4096, 32, math.inf, tk.TK_SCALE_UE8M0, outs["codes4"],
                                     outs["scales4"], None, s) == OK
        assert tk.tk_cast_fp8(x, tk.TK_DTYPE_BF16, 2 * n, 2048, 128, tk.TK_SCALE_UE8M0, outs["ccodes"],
                              outs["cscales"], s) == OK
        assert tk.tk_topk_gate(scores, 300, 256, 8, 8, 4, 1, outs["idx"], outs["gw"], s) == OK
        assert tk.tk_topk_to_pos(outs["idx"], 300, 8, 256, outs["pos"], outs["poff"], s) == OK
        assert tk.tk_moe_reduce(xr, rsd, pd, rwd, r.global_scale, r.tokens, r.k, r.hidden, n_rows,
                                tk.TK_DTYPE_BF16, outs["red"], s) == OK
        assert tk.tk_swiglu_cast_fp8(xl, None, nl, hl, 0, math.inf, tk.TK_SCALE_FP32, outs["lcodes"],
                                     outs["lscales"], None, s) == OK
        assert tk.tk_swiglu_cast_fp4(xl, None, nl, hl // 2, 0, math.inf, tk.TK_SCALE_UE8M0, outs["lcodes4"],
                                     outs["lscales4"], None, s) == OK
        assert tk.tk_cast_fp8(xl, tk.TK_DTYPE_BF16, nl, hl, 0, tk.TK_SCALE_FP32, outs["lccodes"], outs["lcscales"],
                              s) == OK
        assert tk.tk_swiglu_cast_fp8(xs, w[:ns], ns, hs, 96, 10.0, tk.TK_SCALE_UE8M0, outs["scodes"], outs["sscales"],
                                     outs["count"], s) == OK
        assert tk.tk_cast_fp4(xs, tk.TK_DTYPE_BF16, ns, 2 * hs, 96, tk.TK_SCALE_FP32, outs["sccodes"],
                              outs["sccscales"], s) == OK
        assert tk.tk_swiglu_cast_fp8(x2, None, n2, h2, 8704, math.inf, tk.TK_SCALE_FP32, outs["tcodes"],
                                     outs["tscales"], None, s) == OK

    def poison():
        for k, t in outs.items():
            if k == "count":
                t.zero_()
            elif t.dtype.is_floating_point:
                t.fill_(-123.0)
            else:
                t.fill_(77)

    poison()
    work()
    torch.cuda.synchronize()
    eager = {k: t.clone() for k, t in outs.items()}
    assert int(eager["count"].item()) > 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch asks
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        poison()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(t.view(torch.uint8) if t.dtype == torch.bfloat16 else t,
                               eager[k].view(torch.uint8) if t.dtype == torch.bfloat16 else eager[k]), \
                f"replay {rep}: {k} differs from the eager result"
