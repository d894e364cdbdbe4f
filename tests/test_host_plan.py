"""The forward's host-side planner and argument checks under AddressSanitizer
and UBSan, on the CPU.

csrc/attn_plan.h (tile choice, GQA head packing, the split-KV plan and
validate()) is plain C++; tests/host/plan_check.cpp drives it over seeded
random shapes, strides and pointer values and checks the invariants it
lists.  Built here with g++ and -fsanitize=address,undefined, so an
out-of-bounds access, a signed overflow or a bad shift in that code fails
the run, as does a broken invariant.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "plan_check.cpp")


def test_plan_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "plan_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "memory_efficient_tiled_amd", "csrc"), SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
