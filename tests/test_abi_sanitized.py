"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with the sanitizers on its host side only (the GPU code
is unchanged) into _build/, and the ABI tests run against that build in a
child process that preloads the sanitizer runtime: every argument check, error
path and ctypes round trip of tests/test_abi.py then runs instrumented, and
any out-of-bounds access, use after free or undefined behaviour in the host
code aborts the child.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "libsegcausal_san.so")
# host-side instrumentation only: each sanitizer flag is scoped to the host pass
SAN_FLAGS = ["-g", "-shared-libsan",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_abi_suite_under_host_sanitizers():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or sanitizer runtime")
    sys.path.insert(0, ROOT)
    from segment_causal_dit_amd.build import build
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    build(extra=SAN_FLAGS, out=OUT)
    env = dict(os.environ, SEGCAUSAL_LIB=OUT, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
