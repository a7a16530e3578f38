"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/sanitize/build_sanitized.py builds a copy of the library whose host code (argument validation, size queries,
launch set-up) is instrumented, and a C driver that calls every entry point with invalid or empty arguments, each of
which must be rejected with its documented status before any HIP call.  The driver must exit 0 with no sanitizer
report.  (Device code is not instrumented: GPU sanitizers are not used here.)"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_host_code_under_asan_and_ubsan():
    sys.path.insert(0, os.path.join(HERE, "sanitize"))
    import build_sanitized as bs
    try:
        _, driver = bs.build()
    except (RuntimeError, subprocess.CalledProcessError, FileNotFoundError) as e:   # no ROCm toolchain here
        pytest.skip(f"sanitized build unavailable: {e}")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert "all checks passed" in report
