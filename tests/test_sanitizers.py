"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code (CPU
only): the oracle driven over every entry point on small pools
(oracle/sanitize_main.c), and the C ABI's host checks driven with the host
library built with both sanitizers (tests/abi_sanitize_main.c).  A report
from either sanitizer, or an unexpected status, fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text and "LeakSanitizer" not in text, text
    assert r.returncode == 0, text
    return text


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-builtin",
                           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "ska_oracle.c"),
                           os.path.join(ROOT, "oracle", "sanitize_main.c"), "-o", exe, "-lm"])
    assert "ok" in _run(exe)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_host_library_checks_under_sanitizers():
    from long_context_decode_ada_amd import build as B
    ENV["ASAN_OPTIONS"] = "detect_leaks=0"        # (the HIP runtime's own allocations at exit)
    assert "ok" in _run(B.build_abi_sanitized())
