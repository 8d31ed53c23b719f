"""The C ABI from plain C: tests/c_abi/abi_from_c.c is compiled with gcc as
C99 (-Wall -Werror) against include/seqcomp.h, linked with the built
libseqcomp.so, and run.  It checks the host-side entry points only (queries,
validation failures, zero-entry calls), so it needs no GPU."""

import os
import shutil
import subprocess

import pytest

from kv_sequence_compression_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_abi_from_plain_c(tmp_path):
    so = _lib.LIB_PATH
    if not os.path.exists(so):
        pytest.skip("libseqcomp.so is not built")
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(so)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c"), "-o", str(exe), so,
           f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
