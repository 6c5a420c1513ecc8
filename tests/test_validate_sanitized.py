"""The argument checks (fa_validate.cpp) built for the host alone with g++
under AddressSanitizer and UndefinedBehaviorSanitizer, driven by
tests/sanitize/validate_fuzz.cpp: known outcomes plus a sweep of extreme and
random arguments.  Any sanitizer report fails the test.  No GPU needed."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_validate_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fa_validate.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "validate_fuzz.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "VALIDATE_SANITIZED_OK" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
