"""The host plan code (plan.cpp, no HIP calls) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven over a grid of valid, degenerate and out-of-range
descriptors, checking the documented workspace-layout invariants (tests/plan_sanitize.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vggt_global_attention_attn_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "plan_sanitize.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "violations 0" in res.stdout
