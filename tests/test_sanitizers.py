"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; device code is not
instrumented): the oracle, driven on every path by oracle/sanitize_main.c, and the library's
host ABI (argument checks, layouts, error paths) through tests/test_abi_host.py, run against a
host-sanitized build of the library with the sanitizer runtime preloaded."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s) for s in sources)


def test_oracle_under_asan_ubsan():
    os.makedirs(SAN_DIR, exist_ok=True)
    exe = os.path.join(SAN_DIR, "oracle_check")
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("sanitize_main.c", "sage_oracle.c")]
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                           "-std=c11", "-o", exe] + srcs + ["-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "oracle sanitizer run ok" in r.stdout


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_tests_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    from bit_quantized_attention_smooth_amd import build as B
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
    if not _newer(B.SANITIZE_OUT, srcs):
        B.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, SAGE_ATTN_LIBRARY=B.SANITIZE_OUT,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
