"""Concurrent first calls from several host threads: in a fresh process, with
no tk_init beforehand, eight threads each make their first fused call on a
stream of their own at the same time (the per-device set-up runs once, under
its lock, while the others wait); every thread's output must equal the
oracle's."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys, threading
sys.path.insert(0, ROOT)
import numpy as np, torch
import moe_activation_bit_amd as tk
import oracle
from moe_activation_bit_amd import workloads as wl

dev = torch.device("cuda:0")
torch.cuda.init()
w = wl.WORKLOADS["fp8_g128_ue8m0_n32768_h2048"]
jobs = []
for t in range(8):
    rows = range(t * 97, t * 97 + 64 + t)
    x = wl.make_x(w, 1, rows=rows)
    wt = wl.make_w(w, 1)[list(rows)]
    jobs.append((x, wt))
barrier = threading.Barrier(8)
errors = []

def run(t):
    try:
        x, wt = jobs[t]
        n = x.shape[0]
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            xd = torch.from_numpy(x.view(np.int16)).to(dev)
            wd = torch.from_numpy(wt).to(dev)
            codes = torch.empty((n, 2048), dtype=torch.uint8, device=dev)
            scales = torch.empty((n, 16), dtype=torch.uint8, device=dev)
            s.synchronize()
            barrier.wait()
            rc = tk.tk_swiglu_cast_fp8(xd, wd, n, 2048, 128, float("inf"), tk.TK_SCALE_UE8M0, codes, scales, None, s)
            s.synchronize()
        assert rc == tk.TkStatus.TK_OK, rc
        want_c, want_s, _ = oracle.swiglu_cast(x, wt, 128, None, 8, 1)
        assert np.array_equal(codes.cpu().numpy(), want_c), f"thread {t}: codes"
        assert np.array_equal(scales.cpu().numpy(), want_s), f"thread {t}: scales"
    except Exception as e:  # reported by the parent
        errors.append(repr(e))

threads = [threading.Thread(target=run, args=(t,)) for t in range(8)]
for th in threads: th.start()
for th in threads: th.join()
print("errors:", errors)
print("threads ok" if not errors else "threads FAILED")
'''


def test_concurrent_first_calls_from_threads():
    print("[gpu-case] concurrent first calls", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT.replace("ROOT", repr(ROOT), 1)], capture_output=True,
                       text=True, timeout=180, cwd=ROOT)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "threads ok" in r.stdout
