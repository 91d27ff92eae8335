"""Build the package's native libraries in-tree.

libtk.so    -- the HIP kernels and C ABI (hipcc, gfx950)
libsynth.so -- the seeded input generator (plain C)
libstreamceil.so -- plain streaming kernels that measure the HBM ceiling
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Compiler flags for every HIP source:
#  -ffp-contract=off       no fused multiply-add contraction of the y products
#  correctly rounded fp32 division (scale = amax / fmt_max)
#  -packed-fp32-ops off    no v_pk_{add,mul,fma}_f32 in generated code
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
    "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{proc.stdout}")
    return proc.stdout


def build_commands():
    return {
        "libtk.so": [HIPCC] + HIP_FLAGS + ["-o", os.path.join(HERE, "libtk.so"),
                                           os.path.join(CSRC, "tk_swiglu_cast.hip")],
        "libstreamceil.so": [HIPCC] + HIP_FLAGS + ["-o", os.path.join(HERE, "libstreamceil.so"),
                                                   os.path.join(CSRC, "stream_ceiling.hip")],
        "libsynth.so": ["gcc", "-O2", "-fPIC", "-shared", "-o", os.path.join(HERE, "libsynth.so"),
                        os.path.join(CSRC, "synth.c"), "-lm"],
    }


def build(extra=None):
    cmds = list(build_commands().values()) + list(extra or [])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_run, cmds))


if __name__ == "__main__":
    build()
