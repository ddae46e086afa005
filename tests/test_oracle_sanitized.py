"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
its own pin tests, run in a child process against an instrumented build
(every out-of-bounds access, use after free, signed overflow, misaligned or
null access, invalid shift, ... aborts that process)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_codec.py", "tests/test_oracle_quant_pack.py", "tests/test_oracle_gemm_chain.py",
             "tests/test_oracle_boundary.py", "tests/test_oracle_mxfp4.py"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.build(force=True, sanitize=True)
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=runtime, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
