"""Randomized checks of the host-only planner under the address and
undefined-behaviour sanitizers.

`plan_fuzz.cpp` drives validation, the single-problem heuristic and the grouped
heuristic with sizes at and past the library's limits, short and huge leading
dimensions, every base alignment, negative and huge workspaces and random forced
requests, and checks what every accepted plan must satisfy (the chosen kernel
matches the dtype and layout, covers M x N, respects the request, stays within the
workspace, and takes the whole-tile and alignment rules of its schedule). Built
with g++ from the planner's plain C++ source; no GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    build = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "dense_gemm_06_amd", "csrc"), os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
             os.path.join(ROOT, "dense_gemm_06_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    for seed in (1, 2, 3):
        r = subprocess.run([str(exe), str(seed), "200000"], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and "0 invariant failures" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
