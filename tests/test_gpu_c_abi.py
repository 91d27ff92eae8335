"""The C ABI from plain C on the GPU: tests/c_abi/abi_check (built by
__graft_entry__.build()) allocates device buffers through the HIP C API, runs
the fused step (FP8 per-block UE8M0, FP4 per-token with clamp and counter, a
ragged FP8 case), the reduce and the gating, and compares every output byte
with the oracle."""
import os
import subprocess

import pytest

import __graft_entry__ as entry

pytestmark = pytest.mark.gpu


def test_c_program_on_the_gpu():
    assert os.path.exists(entry.C_ABI_CHECK), "tests/c_abi/abi_check is not built: run __graft_entry__.build()"
    print("[gpu-case] c-abi program", flush=True)
    r = subprocess.run([entry.C_ABI_CHECK, "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "c-abi: ok" in r.stdout, r.stdout + r.stderr
