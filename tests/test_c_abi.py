"""The C ABI from C: include/rw4.h compiles as strict C99 and a C program
linked against librw4.so gets the documented status codes (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rotated_w4a4_amd")


def test_c_program_against_the_header(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(PKG, "librw4.so")):
        pytest.skip("librw4.so not built")
    exe = tmp_path / "c_abi_check"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Wpedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", PKG, "-lrw4", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(filter(None, ["/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")]))
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr
