"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The static step plan (``csrc/kd_plan.h``: partitions of rows and FFN slices over workgroups and
waves, the attention split at every position, the exchange-word and row-scale layouts) is plain
integer C++ that the packer and every workgroup repeat. ``tests/host/plan_check.cpp`` includes it
unchanged, checks the properties the kernels rely on over the workload shapes and every cache
position, and is built here with g++ and both sanitizers (host code only; no GPU code is built
with them), so an out-of-bounds access or a signed overflow in the plan fails this test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "bandwidth_bound_transformer_amd", "csrc"),
           "-o", str(exe), os.path.join(ROOT, "tests", "host", "plan_check.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "plan checks passed" in r.stdout
