"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip (argument checks, the Givens / sign table builders, error mapping) is
compiled with the sanitizers on its host side only (``-Xarch_host``: the GPU
code is built as usual), linked with the other objects of the normal build
into a separate library, and driven by two C programs: the C99 header check
and tests/c_abi_sanitize.c (table builders with valid and invalid tables,
every entry point's validation).  No kernel is launched, so this runs
without a GPU.  Leak checking is off: the HIP runtime keeps allocations for
the life of the process.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotated_w4a4_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _host_only(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not available")
    objs = [os.path.join(BUILD, f"{n}.hip.o") for n in ("dequant", "gemm", "quant")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("build the library first (its objects are reused)")
    d = tmp_path_factory.mktemp("asan")
    api_o = d / "api.o"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *_host_only(SAN),
           "-c", os.path.join(CSRC, "api.hip"), "-o", str(api_o)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    lib = d / "librw4.so"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *_host_only(SAN), "-o", str(lib), str(api_o), *objs]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return d


@pytest.mark.parametrize("prog,ok_line", [("c_abi_check.c", "c abi ok"), ("c_abi_sanitize.c", "sanitized host ok")])
def test_host_code_under_sanitizers(sanitized_lib, prog, ok_line):
    d = sanitized_lib
    exe = d / prog.replace(".c", "")
    cmd = [CLANG, "-std=c99", "-g", *SAN, "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", prog),
           "-L", str(d), "-lrw4", f"-Wl,-rpath,{d}", "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(filter(None, ["/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")]))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and ok_line in r.stdout, r.stdout + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
