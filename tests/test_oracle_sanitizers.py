"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/oracle_driver.cpp calls every function of the oracle on small inputs
(batches with a poisoned tensor, subnormal alphas, values near the bf16 maximum,
single blocks, ragged thread splits).  Built with g++ and both sanitizers, with
recovery off, any report ends the program with a nonzero status.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call([
        "g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-pthread",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
        "-I", os.path.join(ROOT, "oracle"),
        "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp"),
        os.path.join(ROOT, "oracle", "nvfp4_oracle.cpp")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "oracle driver: ok" in out, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out
