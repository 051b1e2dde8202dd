"""Host-side checks of the stream-K share arithmetic the kernels use.

`streamk_check.cpp` includes dense_gemm_06_amd/csrc/streamk.h and compares its
double-precision quotient (corrected by one step) with exact integer division, and
its share bounds, owner search and pieces with a plain integer restatement. Built
with hipcc as host code; no GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_streamk_arithmetic(tmp_path):
    exe = tmp_path / "streamk_check"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", os.path.join(ROOT, "tests", "streamk_check.cpp"), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout[-2000:]
