"""The plan builder and the C ABI's argument validation, compiled on the host
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer (plan.cpp and
validate.cpp make no HIP call), run as a native test program."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_05_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_and_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "test_host"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Wextra", "-Wno-unused-parameter",
           os.path.join(ROOT, "tests", "host", "test_host.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "validate.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
