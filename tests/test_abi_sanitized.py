"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_sanitized_check.cpp calls every entry point with arguments the host
validation must refuse (so no GPU is needed), and the error and timing hooks
from eight threads at once; build.build_sanitized_check() compiles it with
the library's sources, the sanitizers on the host code only. A control build
with a planted heap overflow must be stopped by the sanitizer."""
import os
import shutil
import subprocess

import pytest

from draft_token_verification_flattened_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_abi_host_code_is_clean_under_sanitizers():
    exe = build.build_sanitized_check()
    res = _run(exe)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all expectations hold" in res.stdout
    assert "runtime error" not in res.stderr          # UndefinedBehaviorSanitizer reports


def test_sanitizer_stops_a_planted_overflow():
    exe = build.build_sanitized_check(planted=True)
    res = _run(exe)
    assert res.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in res.stderr
