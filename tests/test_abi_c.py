"""The C ABI from plain C (no GPU): include/tk.h compiles as strict C99, and
tests/c_abi/abi_check.c -- a C program that links libtk.so, the input
generator and the oracle -- runs its argument checks: every entry point
rejects bad arguments with the documented status before any HIP call."""
import os
import subprocess

import __graft_entry__ as entry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_is_strict_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "tk.h"\nint main(void) { return tk_status_str(TK_OK) == 0; }\n')
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                    "-I" + os.path.join(ROOT, "include"), str(src)], check=True)


def test_c_program_argument_checks(tmp_path):
    exe = str(tmp_path / "abi_check")
    subprocess.run(entry.c_abi_check_command(exe), check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c-abi: ok" in r.stdout, r.stdout + r.stderr
