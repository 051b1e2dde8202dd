"""Register and scratch budget of every compiled kernel.

The build writes the compiler's per-function resource report
(dense_gemm_06_amd/_build/resource_usage.json). A kernel whose accumulators end
up in scratch memory still computes correct results while running several times
slower, so parity tests cannot catch it: these checks do. Known exceptions are
listed with their exact figures.
"""
import json
import os
import re

import pytest

from dense_gemm_06_amd import build

# the grouped 256 x 256 register-staged kernel with element-wise loads and row-major
# B keeps one register in scratch (8 bytes per lane)
ALLOWED = {re.compile(r"mfma16_gemm_grouped.*Lb0ELi256ELi256ELi64ELi2ELi4E"): (8, 1)}


@pytest.fixture(scope="module")
def usage():
    if not os.path.exists(build.RESOURCE_USAGE):
        build.build()
    with open(build.RESOURCE_USAGE) as f:
        return json.load(f)


def test_report_covers_the_kernels(usage):
    names = " ".join(usage)
    for k in ("mfma16_pp", "mfma16_gemm", "mfma32_gemm", "lds_gemm", "_grouped", "splitk_reduce", "pack_pad"):
        assert k in names, k


def test_no_scratch_or_spills(usage):
    bad = []
    for name, r in usage.items():
        scratch, spill = r.get("ScratchSize [bytes/lane]", 0), r.get("VGPRs Spill", 0)
        allowed = next((v for p, v in ALLOWED.items() if p.search(name)), (0, 0))
        if (scratch, spill) != (0, 0) and (scratch, spill) != allowed:
            bad.append((name, scratch, spill))
    assert not bad, bad


def test_headline_kernels_keep_two_waves_per_simd(usage):
    for pattern in (r"mfma16_ppILi1ELi0ELi16E", r"mfma32_gemmILi0ELb1ELi256ELi128ELi32ELi4ELi2E"):
        r = next(v for k, v in usage.items() if re.search(pattern, k))
        assert r["Occupancy [waves/SIMD]"] == 2 and r["VGPRs"] + r["AGPRs"] <= 256, r
