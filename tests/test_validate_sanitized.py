"""The library's host validation (csrc/isd_validate.cpp) built alone -- it has no HIP
dependency -- with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, and run
through tests/c/validate_test.cpp: valid and invalid calls of every entry point, the
workspace carve-ups, and a deterministic fuzz of the integer arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "strided_verify_propose_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "validate_test"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "c", "validate_test.cpp"), os.path.join(CSRC, "isd_validate.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "validate ok" in res.stdout
