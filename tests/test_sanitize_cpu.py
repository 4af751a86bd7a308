"""The library's host code (budget sizing, argument validation) and the C
oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (every
finding aborts), exercised by tests/sanitize/host_checks.cpp on random and
edge-case inputs.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_verification_spec_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_host_code_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    obj = str(tmp_path / "oracle.o")
    subprocess.check_call(["gcc", *san, "-std=c11", "-c", os.path.join(ROOT, "oracle", "spec_oracle.c"), "-o", obj])
    exe = str(tmp_path / "host_checks")
    subprocess.check_call(["g++", *san, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
                           os.path.join(CSRC, "budget.cpp"), obj, "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
