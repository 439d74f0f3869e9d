"""The CPU tier again with the host code under AddressSanitizer and
UndefinedBehaviorSanitizer: the fp64 oracle (oracle_cev.c, built by clang with
-fsanitize=address,undefined) and the C ABI's host-side argument checks
(api.cpp and noalloc.hip host code in libcevocab_san.so; no device code is
instrumented), loaded with clang's ASan runtime preloaded into a child
pytest.  Any sanitizer report aborts the child (-fno-sanitize-recover)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_cpu_tier_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    from cross_entropy_vocab_amd import build as hip_build
    oracle.build_sanitized()
    lib = hip_build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, CEV_LIBRARY=lib, CEV_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-q",
                        "-p", "no:cacheprovider", "--deselect",
                        "tests/test_host_sanitizers.py::test_cpu_tier_under_asan_and_ubsan"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
