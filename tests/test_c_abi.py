"""The header is plain C: tests/c_abi_check.c, compiled as C99 with every warning an error and
linked against the built library, runs the host-side calls (plan, counts, layout, argument
checks, rejected descriptors) without a GPU."""
import os
import shutil
import subprocess

import pytest

from tests.test_abi_cpu import ROOT, ensure_built


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_program_uses_the_abi(tmp_path):
    va = ensure_built()
    libdir = os.path.dirname(va.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-l:" + os.path.basename(va.LIB_PATH),
           "-Wl,-rpath," + libdir, "-Wl,-rpath-link," + os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "c abi ok"
