"""Build the HIP library libdensegemm.so in-tree, for gfx950 only.

Every translation unit is compiled with hipcc; the kernel families compile in
parallel. Packed-fp32 VALU instructions are disabled for all device code.
Run as ``python -m dense_gemm_06_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdensegemm.so")
ARCH = "gfx950"

DEVICE_SOURCES = ["inst_lds_f32.hip", "inst_lds_f16.hip", "inst_lds_bf16.hip",
                  "inst_mfma_f32.hip", "inst_mfma_f16.hip", "inst_mfma_bf16.hip", "reduce.hip", "pack.hip"]
HOST_SOURCES = ["plan.cpp", "gemm_api.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-gpu-rdc", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    return r.returncode, "\n".join(lines)


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
    failed = [(s, out) for s, rc, out in results if rc != 0]
    for s, rc, out in results:
        if verbose and out.strip():
            print(f"--- {s}\n{out}")
    if failed:
        msg = "\n".join(f"--- {s}\n{out}" for s, out in failed)
        raise RuntimeError(f"HIP build failed:\n{msg}")
    tmp = LIB + ".tmp%d" % os.getpid()
    rc, out = _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[t[1] for t in tasks]])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
