"""The host side of the C ABI under AddressSanitizer and UBSan (no GPU needed).

Builds a copy of the library whose csrc/api.hip host code is instrumented
(build.build_host_sanitized: the argument checks, the plan, the workspace
carving and the launch sequencing; device code as in the normal build) and
runs the host-only ABI tests against it in a child process with the ASan
runtime preloaded.  Any heap or stack overflow, use after free or undefined
behaviour (signed overflow, bad shifts, misaligned or null access) on those
paths aborts the child and fails this test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_13_amd")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_host_paths_clean_under_asan_and_ubsan():
    if not os.path.exists(os.path.join(PKG, "_build", "route.o")):
        pytest.skip("the normal build's objects are missing (run build.py first)")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in the ROCm LLVM tree")
    sys.path.insert(0, PKG)
    import build as B
    lib = B.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, MOE_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
