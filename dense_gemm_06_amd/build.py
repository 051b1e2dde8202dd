"""Build the HIP library libdensegemm.so in-tree, for gfx950 only.

Every translation unit is compiled with hipcc; the kernel families compile in
parallel. Packed-fp32 VALU instructions are disabled for all device code. The
compiler's per-kernel resource usage (registers, scratch, spills, LDS,
occupancy) is written to _build/resource_usage.json.
Run as ``python -m dense_gemm_06_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdensegemm.so")
# Calibration kernels for the HBM traffic counters (a measurement tool, linked apart
# from the GEMM library).
PROBE_LIB = os.path.join(HERE, "libdgprobe.so")
ARCH = "gfx950"

DEVICE_SOURCES = ["inst_lds_f32.hip", "inst_lds_f16.hip", "inst_lds_bf16.hip",
                  "inst_mfma_f32.hip", "inst_mfma_f16.hip", "inst_mfma_bf16.hip", "reduce.hip", "pack.hip",
                  "noalloc.hip"]
HOST_SOURCES = ["plan.cpp", "gemm_api.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]
# Loops start on a 64-byte boundary: the fp32 256 x 128 direct-copy kernel with
# row-major B ran its steady-state loop 17% slower with the loop head at byte 28 of a
# 64-byte line (4096^3: 1179 us) than at byte 52 (1011) or aligned (1010-1011), with the
# same instructions; the padding keeps a prologue edit from moving a kernel's speed.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-falign-loops=64", "-fno-gpu-rdc", "-munsafe-fp-atomics", "-Rpass-analysis=kernel-resource-usage"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


RESOURCE_USAGE = os.path.join(OUT_DIR, "resource_usage.json")
_REMARK = re.compile(r"remark: (.*?) \[-Rpass-analysis=kernel-resource-usage\]")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless;
    # resource-usage remarks are collected separately
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l
             and "kernel-resource-usage" not in l and not l.lstrip().startswith(("|", "^"))
             and not re.match(r"^\s*\d+ \|", l)]
    return r.returncode, "\n".join(lines), r.stdout


def _resource_usage(text: str) -> dict:
    """Per device function: the compiler's resource-usage remarks (VGPRs, AGPRs,
    scratch bytes per lane, spills, LDS, occupancy)."""
    out, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        t = m.group(1).strip()
        if t.startswith("Function Name:"):
            cur = out.setdefault(t.split(":", 1)[1].strip(), {})
        elif cur is not None and ":" in t:
            k, v = t.split(":", 1)
            v = v.strip()
            cur[k.strip()] = int(v) if v.lstrip("-").isdigit() else v
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link LIB. Always recompiles (a fresh build each call)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    tasks = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        tasks.append((src, obj, [cc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".cpp", ".o"))
        tasks.append((src, obj, [cc, *COMMON, "-x", "hip", f"--offload-arch={ARCH}", "--cuda-host-only",
                                 "-c", os.path.join(CSRC, src), "-o", obj]))
    jobs = jobs or min(len(tasks), max(1, min(os.cpu_count() or 1, 8)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda t: (t[0], *_run(t[2])), tasks))
    failed = [(s, out) for s, rc, out, _ in results if rc != 0]
    for s, rc, out, _ in results:
        if verbose and out.strip():
            print(f"--- {s}\n{out}")
    usage = {}
    for s, rc, out, raw in results:
        usage.update(_resource_usage(raw))
    with open(RESOURCE_USAGE, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{out}" for s, out in failed)
        raise RuntimeError(f"HIP build failed:\n{msg}")
    tmp = LIB + ".tmp%d" % os.getpid()
    rc, out, _ = _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[t[1] for t in tasks]])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    rc, out, _ = _run([cc, *COMMON, *DEVICE_FLAGS, "-shared", os.path.join(CSRC, "probe.hip"), "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"probe library build failed:\n{out}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
