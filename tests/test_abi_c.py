"""The library from plain C (CPU): a C program that includes only include/isd.h compiles
with gcc, links libisd.so, and its host-side checks pass."""
import os
import shutil
import subprocess

import pytest

from strided_verify_propose_amd.build import LIB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_caller(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libisd.so not built")
    exe = tmp_path / "abi_smoke"
    src = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                    "-o", str(exe), "-L", libdir, "-lisd", f"-Wl,-rpath,{libdir}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "c abi ok" in res.stdout
