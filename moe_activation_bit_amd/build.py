"""Build the package's native libraries in-tree.

libtk.so    -- the HIP kernels and C ABI (hipcc, gfx950; one object per source)
libsynth.so -- the seeded input generator (plain C)
libstreamceil.so -- plain streaming kernels that measure the HBM ceiling
_tkpy            -- the CPython extension behind the Python binding (gcc)
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


OBJ_DIR = os.path.join(HERE, "_build")
TK_SOURCES = ["tk_swiglu_cast.hip", "tk_cast.hip", "tk_topk.hip", "tk_reduce.hip", "tk_pos.hip"]


def _hip_object(src):
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    return obj, [HIPCC] + [f for f in HIP_FLAGS if f != "-shared"] + ["-c", "-o", obj, os.path.join(CSRC, src)]


def build_commands():
    """(stage 1 commands that run in parallel, stage 2 link commands)"""
    objs = [_hip_object(s) for s in TK_SOURCES]
    stage1 = [cmd for _, cmd in objs] + [
        [HIPCC] + HIP_FLAGS + ["-o", os.path.join(HERE, "libstreamceil.so"), os.path.join(CSRC, "stream_ceiling.hip")],
        ["gcc", "-O2", "-fPIC", "-shared", "-o", os.path.join(HERE, "libsynth.so"), os.path.join(CSRC, "synth.c"),
         "-lm"],
    ]
    stage2 = [[HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", os.path.join(HERE, "libtk.so")]
              + [o for o, _ in objs], extension_command()]
    return stage1, stage2


def extension_command():
    """gcc line for the CPython extension _tkpy (argument marshalling to
    libtk.so, found next to it at run time)."""
    import sysconfig
    out = os.path.join(HERE, "_tkpy" + sysconfig.get_config_var("EXT_SUFFIX"))
    return ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra", "-Werror",
            "-I" + sysconfig.get_paths()["include"], "-I" + os.path.join(ROOT, "include"),
            os.path.join(CSRC, "tk_py.c"), "-o", out, "-L" + HERE, "-ltk", "-Wl,-rpath,$ORIGIN"]


def build(extra=None):
    os.makedirs(OBJ_DIR, exist_ok=True)
    stage1, stage2 = build_commands()
    cmds = stage1 + list(extra or [])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_run, cmds))
    for cmd in stage2:
        _run(cmd)


if __name__ == "__main__":
    build()
