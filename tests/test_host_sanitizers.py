"""The C ABI's host-side argument handling (attn_api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

attention_forward_06_amd/csrc/host_checks.cpp drives every entry point with fake device pointers
against a stub launcher: boundary sizes and strides at the int64 extremes, misaligned pointers
and strides, and 200k seeded random calls.  Built here with g++ (host code only, no HIP), so any
signed overflow, bad shift or out-of-bounds access in the checks aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_forward_06_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "host_checks.cpp"), os.path.join(CSRC, "attn_api.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)   # the sanitizer runtime must be the first library loaded
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host checks passed" in run.stdout
    assert "runtime error" not in run.stderr
