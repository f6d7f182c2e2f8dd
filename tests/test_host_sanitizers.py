"""The host side of the C ABI (argument checks, size arithmetic, dispatch) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU: fa_api.cpp is rebuilt with both (host code only; the
kernels are the ordinary objects) and every case of test_lib_cpu.py -- argument errors at the
int32 limits, empty batches, the decode chunk override, the allocation-free entry point's size
check -- runs against it in a child process that preloads the sanitizer runtime. Any report
aborts the child (UBSan without recovery, ASan halting on the first error). No kernel is
launched."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_argument_checks_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from io_aware_exact_23_amd import build as fab

    lib = fab.build_host_sanitized()
    env = dict(os.environ)
    env.update(FA_TEST_LIBRARY=lib, LD_PRELOAD=fab.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("FA_DECODE_CHUNK", None)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_lib_cpu.py"),
                        "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert " passed" in r.stdout, out
