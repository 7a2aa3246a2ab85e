"""The host tests again, against the host C++ built with AddressSanitizer and
UndefinedBehaviorSanitizer (liboscar_san.so: pool, planner, calibration and
argument checks instrumented; device objects unchanged).  They run in a
child process with clang's ASan runtime preloaded; any sanitizer report
aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

from kv_cache_int2_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import kv_cache_int2_amd as K
assert K.LIB_PATH.endswith("liboscar_san.so"), K.LIB_PATH
K.lib()
maps = open("/proc/self/maps").read()
assert "liboscar_san.so" in maps and "libclang_rt.asan" in maps, "sanitized library not loaded"
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_host.py"]))
"""


def test_host_tests_pass_under_asan_and_ubsan():
    try:
        lib = B.build_sanitized()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = dict(os.environ, OSCAR_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
