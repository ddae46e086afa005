"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: argument validation, the GEMM planner, the
workspace and scratch size arithmetic and the plan sweeps of the host ABI
tests, run in a child process against libvla_san.so, a build whose host code
is instrumented (every out-of-bounds access, use after free, signed
overflow, invalid shift, misaligned or null access aborts that process).
No kernel is launched."""
import glob
import os
import subprocess
import sys

import pytest

from bf16_gemm_vla_amd import build as vla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_under_asan_and_ubsan():
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = vla_build.build(sanitize=True)
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout and "__ubsan_handle" in nm.stdout, "host code is not instrumented"
    runner = ("import sys; sys.path.insert(0, %r)\n"
              "import bf16_gemm_vla_amd._lib as L; L.LIB_PATH = %r\n"
              "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
              "'tests/test_abi_host.py']))\n") % (ROOT, lib)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
