#!/usr/bin/env python3
"""Benchmark of the MI355X dense GEMM C = A @ B (one GPU).

One step is one C = A @ B over the 4096^3 fp16-input / fp32-accumulate problem
(row-major A and B, fp32 C; entries uniform[-1, 1) rounded to fp16, seed 0),
launched through the library's C ABI in the configuration its heuristic picks.
The fp32 4096^3 problem (the other half of the headline metric) and the other
benchmark shapes are timed the same way and reported alongside.

Timing: W untimed warm-up steps, then exactly K steps back to back, bracketed by
torch.cuda.synchronize(); the duration is taken from HIP events recorded on the
launch stream around the K launches. One kernel runs per step and the launches
follow each other with no gap, so the step time is also the kernel's average
duration (the roofline figure). Inputs are resident in HBM before timing starts.
The other problems are timed the same way over K/2 steps or more, after a
warm-up of about 20 ms of their launches (the clock rises over the first
milliseconds of sustained work): a small problem gets enough steps for about 5 ms
of launches (reported as `steps`), so that the start of the idle queue, paid once
per timed window, does not weigh on its step time.

Only the W + K headline launches run the headline kernel on its 256-workgroup grid
in the default command (the fused epilogue, the per-launch distribution and the
clock probe, which launch it many more times, run only with --extended; the K-split
launches of the 512 x 4096 x 4096 shard run the same kernel on a 2-D grid), so a
kernel trace of the default command, filtered by grid, averages exactly those
launches.

CPU baseline: the oracle (plain fp64 triple loop, OpenMP) timed on the host
cores on a bounded sample of the same problem (its first r rows; about 10-20 s
of CPU work), reported as TFLOP/s of the sample.

Prints one JSON line. --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}   # MI355X dense matrix peaks
HBM_GBPS = 8000.0
def kernel_sources(cfg) -> list[str]:
    """The source files a configuration's device code is built from."""
    common = ["device_common.h", "lds_layout.h"]
    if cfg.variant == 1:
        return common + ["kernel_lds.h"]
    if cfg.schedule in (2, 4):
        return common + ["kernel_pp.h"]
    if cfg.schedule in (5, 7):
        return common + ["kernel_sp.h"]
    if cfg.schedule in (8, 9):
        return common + ["kernel_sp.h", "kernel_f32dc.h"]
    return common + ["kernel_mfma.h"]


def kernel_source_hash(cfg) -> str:
    """Hash of a configuration's kernel sources and the device compiler flags (code
    placement alone has changed a kernel's speed)."""
    from dense_gemm_06_amd.build import DEVICE_FLAGS
    h = hashlib.sha256(" ".join(DEVICE_FLAGS).encode())
    for f in kernel_sources(cfg):
        with open(os.path.join(ROOT, "dense_gemm_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="time only the headline problem")
    p.add_argument("--only", default=None, help="time only this benchmark problem, or grouped workload (for profiling)")
    p.add_argument("--force", default=None, metavar="KEY=V,...",
                   help="with --only: force a configuration (gemm_config input fields, e.g. variant=1 or "
                        "schedule=5,waves_n=2), for profiling a kernel the heuristic does not pick")
    p.add_argument("--with-workspace", action="store_true",
                   help="with --only: pass a workspace (the heuristic may split K or pack the operands)")
    p.add_argument("--extended", action="store_true",
                   help="also time the fused epilogue, the per-launch distribution, the clock under load and the "
                        "four-round problem with one workgroup per tile (more launches of the headline kernel, so a "
                        "kernel trace of such a run averages over more than the timed steps)")
    p.add_argument("--mfma-ceiling", action="store_true",
                   help="time libdgprobe.so's MFMA-only loop (every CU, no memory traffic) on changing random fp16 "
                        "operands and on fixed ones: the power-limited ceiling of the 16-bit product")
    p.add_argument("--traffic-probe", type=int, default=0, metavar="MIB",
                   help="instead of GEMMs, run the counter-calibration kernels over MIB MiB each (direct LDS "
                        "copies of 64-byte row segments, 16-byte loads, 16-byte stores)")
    return p.parse_args()


def device_problem(name, seed=0):
    import torch
    import gemm_inputs as gi
    ops = gi.make_config(name, seed=seed)
    def dev(a):
        import numpy as np
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        return t.to("cuda")
    A, B = dev(ops.A), dev(ops.B)
    C = torch.empty((ops.M, ops.N), dtype=torch.float32, device="cuda")
    return ops, A, B, C


WORKSPACE_CAP = 256 << 20   # workspace offered to split-K runs


def time_problem(name, steps, warmup, workspace=False, force=None, min_window_ms=0.0, min_warm_ms=0.0):
    """Warm up, then time exactly `steps` calls with HIP events on the launch stream.

    workspace=True runs gemm_ex_workspace with up to WORKSPACE_CAP bytes (the
    heuristic may split K or pack the operands; such a call is two kernels, both
    inside the timed step). min_window_ms > 0 raises `steps` until the timed
    launches span about that long (estimated from the warm-up), so that the start of
    an idle queue, paid once per timed window, is spread over enough launches of a
    small problem. min_warm_ms > 0 extends the untimed warm-up to about that long:
    the chip raises its clock over the first milliseconds of sustained work (a
    1024^3 fp32 launch measured 24.6 us over the first 20 launches and 22.6 over
    launches 320-420 of one run), which a warm-up of a few short launches does not
    cover."""
    import torch
    import dense_gemm_06_amd as dg
    ops, A, B, C = device_problem(name)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    args = (dg.GEMM_OP_N, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
            C.data_ptr(), ops.N, dg.DTYPE_CODE[ops.dtype])
    cus, arch = dg.gemm_device_info(0)
    req = dg.request(**force) if force else None
    _, cfg = dg.gemm_plan_workspace(args[0], args[1], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ops.N, args[-1],
                                    A.data_ptr(), B.data_ptr(), C.data_ptr(), cus, arch,
                                    WORKSPACE_CAP if workspace else 0, req)
    if workspace and cfg.workspace_bytes > 0:
        W = torch.empty(cfg.workspace_bytes // 4, dtype=torch.float32, device="cuda")
        call = lambda: dg.gemm_ex_workspace(*args, req, W.data_ptr(), cfg.workspace_bytes, s)
    else:
        call = lambda: dg.gemm_ex(*args, req, s)
    t0 = time.perf_counter()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    if (min_window_ms > 0 or min_warm_ms > 0) and warmup > 0:
        per_call_ms = (time.perf_counter() - t0) * 1e3 / warmup
        steps = max(steps, min(4000, int(min_window_ms / max(per_call_ms, 1e-4)) + 1))
        more = min(20000, int(min_warm_ms / max(per_call_ms, 1e-4)) - warmup)
        for _ in range(max(0, more)):
            call()
        torch.cuda.synchronize()
    # whole job: K launches back to back between two events
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # One kernel per step and no host work between launches: a kernel trace of this
    # loop shows the launches back to back with no gap, so the step time is also the
    # kernel's average duration over the timed launches. (Launches separated by
    # idle time run faster: the chip's clock is higher before sustained load.)
    launch_ms = ms
    flops = 2.0 * ops.M * ops.N * ops.K
    del A, B, C
    return dict(problem=name, steps=steps, ms_per_step=ms, launch_ms=launch_ms, tflops=flops / (ms * 1e-3) / 1e12,
                kernel_tflops=flops / (launch_ms * 1e-3) / 1e12, wall_s=wall, dtype=ops.dtype,
                M=ops.M, N=ops.N, K=ops.K, op_b=ops.op_b, flops=flops, cfg=cfg, cus=cus, arch=arch,
                peak=PEAK_TFLOPS[ops.dtype])


def time_fused_epilogue(name, steps, warmup):
    """The problem with a fused epilogue: C = gelu(A @ B + bias) stored as bf16."""
    import numpy as np
    import torch
    import dense_gemm_06_amd as dg
    ops, A, B, _ = device_problem(name)
    C = torch.empty((ops.M, ops.N), dtype=torch.bfloat16, device="cuda")
    bias = torch.from_numpy(np.random.default_rng(1).standard_normal(ops.N).astype(np.float32)).cuda()
    epi = dg.epilogue(bias=bias.data_ptr(), activation="gelu_tanh", out_dtype="bf16")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    args = (0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
            C.data_ptr(), ops.N, dg.DTYPE_CODE[ops.dtype], epi, None, None, 0, s)
    cus, arch = dg.gemm_device_info(0)
    _, cfg = dg.gemm_plan_workspace(0, args[1], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ops.N, args[11],
                                    A.data_ptr(), B.data_ptr(), C.data_ptr(), cus, arch, 0, epi=epi)
    for _ in range(warmup):
        dg.gemm_ex_epilogue(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        dg.gemm_ex_epilogue(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * ops.M * ops.N * ops.K
    return dict(ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12, cfg=cfg, peak=PEAK_TFLOPS[ops.dtype])


# Grouped workloads: `count` independent problems of one shape, run as one grouped
# launch (the README's grouped example: four 256^3 fp32 GEMMs).
GROUPED = {"g4_f32_256": dict(count=4, M=256, N=256, K=256, dtype="f32")}


def time_grouped(name, steps, warmup):
    """One step = every problem of the group in one gemm_grouped call; the same
    problems as separate gemm_ex launches are timed alongside for comparison."""
    import torch
    import numpy as np
    import dense_gemm_06_amd as dg
    import gemm_inputs as gi
    spec = GROUPED[name]
    dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    ops = [gi.make_operands(spec["M"], spec["N"], spec["K"], spec["dtype"], "uniform", seed=s)
           for s in range(spec["count"])]
    bufs = [(dev(o.A), dev(o.B), torch.empty((o.M, o.N), dtype=torch.float32, device="cuda")) for o in ops]
    probs = [dg.problem(o.M, o.N, o.K, A.data_ptr(), o.lda, B.data_ptr(), o.ldb, C.data_ptr(), o.N)
             for o, (A, B, C) in zip(ops, bufs)]
    code = dg.DTYPE_CODE[spec["dtype"]]
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    _, cfg = dg.gemm_grouped_plan(0, 0, code, probs)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: dg.gemm_grouped(0, 0, code, probs, None, s))
    ms_sep = timed(lambda: [dg.gemm_ex(0, 0, o.M, o.N, o.K, A.data_ptr(), o.lda, B.data_ptr(), o.ldb,
                                       C.data_ptr(), o.N, code, None, s) for o, (A, B, C) in zip(ops, bufs)])
    flops = 2.0 * spec["count"] * spec["M"] * spec["N"] * spec["K"]
    return dict(problem=name, ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12, separate_ms=ms_sep,
                separate_tflops=flops / (ms_sep * 1e-3) / 1e12, cfg=cfg, peak=PEAK_TFLOPS[spec["dtype"]])


def sclk_under_load(name, seconds=2.0):
    """The graphics clock while the problem's kernel runs back to back: launches in
    batches for about `seconds`, while a child amd-smi process reads the clock of
    every XCD once, half-way through. Reported as not measured when amd-smi is
    missing or its output cannot be read."""
    import shutil
    import subprocess
    import threading
    import torch
    import dense_gemm_06_amd as dg
    exe = shutil.which("amd-smi")
    if exe is None:
        return {"measured": False, "reason": "amd-smi not found"}
    ops, A, B, C = device_problem(name)
    s = torch.cuda.current_stream().cuda_stream
    call = lambda: dg.gemm_ex(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, A.data_ptr(), ops.lda, B.data_ptr(),
                              ops.ldb, C.data_ptr(), ops.N, dg.DTYPE_CODE[ops.dtype], None, s)
    result = {}

    def probe():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run([exe, "metric", "-c", "-p", "--json"], capture_output=True, text=True, timeout=30)
            data = json.loads(r.stdout)
            gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
            clocks = {k: v["clk"]["value"] for k, v in gpu["clock"].items() if k.startswith("gfx_")}
            result.update(measured=True, source="amd-smi metric -c -p", workload=name,
                          mhz_per_xcd=list(clocks.values()), mhz_mean=round(sum(clocks.values()) / len(clocks), 1),
                          mhz_max_rated=max(v["max_clk"]["value"] for k, v in gpu["clock"].items()
                                            if k.startswith("gfx_")))
            try:
                result["socket_power_w"] = gpu["power"]["socket_power"]["value"]
            except (KeyError, TypeError):
                pass
        except Exception as exc:  # the clock is context; the run goes on without it
            result.update(measured=False, reason=f"{type(exc).__name__}: {str(exc)[:160]}")
        smi = shutil.which("rocm-smi")
        if smi:
            try:  # the board's power cap, when the tool reports it
                r = subprocess.run([smi, "--showmaxpower", "--json"], capture_output=True, text=True, timeout=30)
                card = next(iter(json.loads(r.stdout).values()))
                cap = [v for k, v in card.items() if "power" in k.lower()]
                if cap:
                    result["power_cap_w"] = float(str(cap[0]).split()[0])
            except Exception:
                pass

    t = threading.Thread(target=probe)
    t.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or t.is_alive():
        for _ in range(50):
            call()
        torch.cuda.synchronize()
    t.join()
    del A, B, C
    return result


def time_distribution(name, n=100, warmup=10, n_cold=10, cold_bytes=512 << 20):
    """Per-launch durations: n launches back to back with an event pair around each
    (median, min, max), and n_cold launches each preceded by a write of cold_bytes
    of scratch, which evicts the inputs from the 256 MB MALL ("cold")."""
    import torch
    import dense_gemm_06_amd as dg
    ops, A, B, C = device_problem(name)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    call = lambda: dg.gemm_ex(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, A.data_ptr(), ops.lda, B.data_ptr(),
                              ops.ldb, C.data_ptr(), ops.N, dg.DTYPE_CODE[ops.dtype], None, s)
    for _ in range(warmup):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    warm = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
    scratch = torch.empty(cold_bytes // 4, dtype=torch.float32, device="cuda")
    cold = []
    for i in range(n_cold):
        scratch.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    cold.sort()
    del scratch, A, B, C
    flops = 2.0 * ops.M * ops.N * ops.K
    med = lambda v: v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    return {"warm": {"launches": n, "median_us": round(med(warm), 2), "min_us": round(warm[0], 2),
                     "max_us": round(warm[-1], 2), "tflops_at_median": round(flops / (med(warm) * 1e-6) / 1e12, 1),
                     "tflops_at_min": round(flops / (warm[0] * 1e-6) / 1e12, 1)},
            "cold": {"launches": n_cold, "evict_bytes": cold_bytes, "median_us": round(med(cold), 2),
                     "min_us": round(cold[0], 2), "tflops_at_median": round(flops / (med(cold) * 1e-6) / 1e12, 1)}}


def cpu_small(name, rows=None):
    """The oracle on c1 / c2 with all host threads and with one thread (GFLOP/s); a
    bounded row sample for the larger one."""
    import gemm_inputs as gi
    import oracle
    ops = gi.make_config(name)
    oracle.build(force=False)
    rows = list(range(rows or ops.M))
    out = {}
    cores = oracle.max_threads()
    for label, nt in (("all_threads", 0), ("one_thread", 1)):
        _, t = oracle.timed_gemm_ref(ops, rows=rows, nthreads=nt)
        out[label] = round(2.0 * len(rows) * ops.N * ops.K / t / 1e9, 3)
    out.update(unit="GFLOP/s", cores=cores, kind="oracle",
               sample=f"rows 0..{len(rows) - 1} of {ops.M}x{ops.N}x{ops.K} {ops.dtype}")
    return out


def cpu_baseline(name, target_s):
    """The oracle on the first r rows of `name`, r chosen for about target_s seconds."""
    import gemm_inputs as gi
    import oracle
    ops = gi.make_config(name)
    oracle.build(force=False)
    # calibrate: the per-call fixed cost (decoding B) cancels in the difference
    _, t1 = oracle.timed_gemm_ref(ops, rows=list(range(16)))
    _, t2 = oracle.timed_gemm_ref(ops, rows=list(range(48)))
    per_row = max((t2 - t1) / 32, 1e-5)
    r = int(max(16, min(ops.M, target_s / per_row)))
    _, t = oracle.timed_gemm_ref(ops, rows=list(range(r)))
    flops = 2.0 * r * ops.N * ops.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"rows 0..{r - 1} of the {ops.M}x{ops.N}x{ops.K} {ops.dtype} problem "
                      f"({r / ops.M:.4f} of its work), Cref only, fp64 accumulation; {t:.2f} s",
            "seconds": t, "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_name(cfg, dtype):
    """The kernel template a configuration launches (as named in the rocprofv3 traces)."""
    if cfg.variant == 1:
        base = "lds_gemm"
    elif dtype == "f32":
        base = ("mfma32_gemm, three LDS stages" if cfg.schedule == 6 else
                "mfma32_dc, direct copies" if cfg.schedule == 8 else
                "mfma32_dcl, direct copies" if cfg.schedule == 9 else "mfma32_gemm")
    else:
        base = {1: "mfma16_gemm", 2: "mfma16_pp (16x16x32)", 4: "mfma16_pp (32x32x16)",
                5: "mfma32_sp (32x32x16)", 7: "mfma32_sp, register-staged (32x32x16)"}[cfg.schedule]
    if cfg.grid < cfg.tiles_total:
        base += f", persistent grid of {cfg.grid}"
    return f"{base} {cfg.bm}x{cfg.bn}x{cfg.bk} waves {cfg.waves_m}x{cfg.waves_n}"


def load_traffic(problem, cfg):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this kernel build."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(problem)
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(cfg) or rec.get("kernel_id") != cfg.kernel_id:
        return None
    return rec.get("hbm_bytes_per_launch")


def traffic_probe(mib):
    """One launch of each calibration kernel of libdgprobe.so over `mib` MiB: the bytes
    each moves are known, so a counter run over this command gives the counter-to-bytes
    factor of each memory form (probe_read_lds, probe_read_vec, probe_write)."""
    import ctypes
    import torch
    from dense_gemm_06_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.dg_probe_traffic.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.dg_probe_out_bytes.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.dg_probe_out_bytes.restype = ctypes.c_int64
    nbytes = mib << 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(max(lib.dg_probe_out_bytes(k, nbytes) for k in (0, 1)) // 4 + 1, dtype=torch.int32,
                      device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    res = {}
    for kind, name in ((0, "probe_read_lds"), (1, "probe_read_vec"), (2, "probe_write")):
        rc = lib.dg_probe_traffic(kind, src.data_ptr(), dst.data_ptr() if kind == 2 else out.data_ptr(), nbytes, s)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"{name}: status {rc}")
        res[name] = {"bytes_read" if kind < 2 else "bytes_written": nbytes}
    print(json.dumps({"traffic_probe": res}), flush=True)


def mfma_ceiling(cus, iters=20000, reps=10):
    """TFLOP/s of libdgprobe.so's MFMA-only loop on all compute units, after three
    untimed launches, for operand fragments drawn uniform in [-1, 1) (as the benchmark's
    fp16 inputs), all 0.5, and all zero."""
    import ctypes
    import numpy as np
    import torch
    from dense_gemm_06_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.dg_probe_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.dg_probe_mfma_frag_bytes.restype = ctypes.c_int64
    lib.dg_probe_mfma_out_bytes.argtypes = [ctypes.c_int]
    lib.dg_probe_mfma_out_bytes.restype = ctypes.c_int64
    n = lib.dg_probe_mfma_frag_bytes() // 2
    out = torch.empty(lib.dg_probe_mfma_out_bytes(cus) // 4, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    rng = np.random.default_rng(0)
    for name, vals in (("random_uniform", rng.uniform(-1.0, 1.0, n)), ("constant_0.5", np.full(n, 0.5)),
                       ("zero", np.zeros(n))):
        frag = torch.from_numpy(vals.astype(np.float16)).to("cuda")
        run = lambda: lib.dg_probe_mfma_ceiling(frag.data_ptr(), out.data_ptr(), cus, iters, s)
        for _ in range(3):
            if run() != 0:
                raise RuntimeError("probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = cus * 8 * iters * 64 * 32768.0
        res[name] = {"ms_per_launch": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["f16"], 4)}
    print(json.dumps({"mfma_ceiling": res, "cus": cus, "iters": iters, "launches": reps}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if a.traffic_probe:
        traffic_probe(a.traffic_probe)
        return
    if a.mfma_ceiling:
        mfma_ceiling(torch.cuda.get_device_properties(0).multi_processor_count)
        return
    import dense_gemm_06_amd as dg
    dg.library()   # fail loudly if the HIP library is missing

    if a.only in GROUPED:
        r = time_grouped(a.only, a.steps, a.warmup)
        print(json.dumps({k: (v.as_dict() if k == "cfg" else v) for k, v in r.items()}), flush=True)
        return
    headline = a.only or "c4_f16_4096"
    force = None
    if a.force:
        if not a.only:
            print("--force needs --only", file=sys.stderr)
            sys.exit(2)
        force = {k: int(v) for k, v in (kv.split("=") for kv in a.force.split(","))}
    main_res = time_problem(headline, a.steps, a.warmup, workspace=bool(a.only and a.with_workspace), force=force)
    # the fused-epilogue variant right after the headline, in the same thermal state
    # (the chip's clock drifts by 10-20% over a run of heavy launches)
    fe = None
    if a.extended and not a.only:
        fe = time_fused_epilogue(headline, max(5, a.steps // 2), max(2, a.warmup // 2))
    extras = {}
    if not a.no_extra and not a.only:
        for name in ("c3_f32_4096", "c1_f32_256", "c2_f32_1024", "c5_bf16_ragged", "m8_f16_shard", "m8_f32_shard",
                     "r4_f16_8192x8192x2048", "t33_f16_4352x4352x2048"):
            extras[name] = time_problem(name, max(5, a.steps // 2), max(2, a.warmup // 2), min_window_ms=5.0, min_warm_ms=20.0)
        # the same four-round problem with one workgroup per tile (no persistent grid):
        # the headline's kernel, so only with --extended (the default command runs the
        # headline kernel for the headline's steps alone)
        one_per_tile = None
        if a.extended:
            one_per_tile = time_problem("r4_f16_8192x8192x2048", max(5, a.steps // 2), max(2, a.warmup // 2),
                                        force={"max_grid": 1 << 30}, min_window_ms=5.0, min_warm_ms=20.0)

    cfg = main_res["cfg"]
    traffic = load_traffic(headline, cfg)
    import gemm_inputs as gi
    spec = gi.CONFIGS.get(headline) or gi.EXTRA_CONFIGS[headline]
    dist_text = "uniform[-1,1)" if spec["dist"] == "uniform" else "normal N(0,1)"
    b_text = "row-major" if spec["op_b"] == "N" else "column-major"
    roof = {"bound": "mfma", "achieved": main_res["kernel_tflops"], "peak": main_res["peak"], "unit": "TFLOP/s",
            "frac": main_res["kernel_tflops"] / main_res["peak"], "traffic": traffic,
            "kernel": kernel_name(cfg, main_res["dtype"]),
            "flops_per_launch": main_res["flops"], "launch_ms": main_res["launch_ms"]}
    out = {
        "metric": "GEMM TFLOP/s (2MNK/t) at 4096^3 fp16-in/fp32-acc (value) and fp32 (fp32 field); % of MFMA peak",
        "value": round(main_res["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": f"synthetic (seeded {dist_text} rounded to the input dtype)",
        "config": {"workload": f"C=A@B {main_res['M']}x{main_res['N']}x{main_res['K']} {main_res['dtype']} in, "
                               f"fp32 acc/out, row-major A, {b_text} B", "M": main_res["M"], "N": main_res["N"],
                   "K": main_res["K"], "kernel_cfg": {k: v for k, v in cfg.as_dict().items() if k != "est_cycles"},
                   "cus": main_res["cus"], "arch": main_res["arch"]},
        "pct_of_peak": round(100 * main_res["tflops"] / main_res["peak"], 2),
        "roofline": roof,
    }
    if "c3_f32_4096" in extras:
        r = extras["c3_f32_4096"]
        out["fp32"] = {"value": round(r["tflops"], 3), "unit": "TFLOP/s", "ms_per_step": round(r["ms_per_step"], 6),
                       "peak": r["peak"], "frac": r["tflops"] / r["peak"],
                       "roofline": {"bound": "mfma", "achieved": r["kernel_tflops"], "peak": r["peak"],
                                    "unit": "TFLOP/s", "frac": r["kernel_tflops"] / r["peak"],
                                    "traffic": load_traffic("c3_f32_4096", r["cfg"]),
                                    "kernel": kernel_name(r["cfg"], r["dtype"]), "launch_ms": r["launch_ms"]},
                       "kernel_cfg": {k: v for k, v in r["cfg"].as_dict().items() if k != "est_cycles"}}
    if extras:
        out["other_problems"] = {k: {"tflops": round(v["tflops"], 3), "ms_per_step": round(v["ms_per_step"], 6),
                                     "steps": v["steps"],
                                     "frac_of_peak": round(v["tflops"] / v["peak"], 4),
                                     "tile": f"{v['cfg'].bm}x{v['cfg'].bn}",
                                     "variant": "mfma" if v["cfg"].variant == 2 else "lds"}
                                 for k, v in extras.items()}
        for k, v in extras.items():
            out["other_problems"][k]["grid"] = v["cfg"].grid
        out["other_problems"]["r4_f16_8192x8192x2048"]["workload"] = (
            "C=A@B 8192x8192x2048 f16: four rounds of 256 tiles on the persistent grid")
        out["other_problems"]["t33_f16_4352x4352x2048"]["workload"] = (
            "C=A@B 4352x4352x2048 f16: a round of 256 tiles and a tail of 33 (with a workspace: stream-K)")
        if one_per_tile is not None:
            r = one_per_tile
            out["other_problems"]["r4_f16_8192x8192x2048"]["one_workgroup_per_tile"] = {
                "tflops": round(r["tflops"], 3), "ms_per_step": round(r["ms_per_step"], 6), "grid": r["cfg"].grid}
        # the under-filled problems again with a workspace (the heuristic may split K),
        # and a long-K problem with 16 output tiles, where splitting pays
        lk = time_problem("k1_f32_long_k", max(5, a.steps // 2), max(2, a.warmup // 2), min_window_ms=5.0, min_warm_ms=20.0)
        out["other_problems"]["k1_f32_long_k"] = {
            "workload": "C=A@B 256x256x16384 f32", "tflops": round(lk["tflops"], 3),
            "ms_per_step": round(lk["ms_per_step"], 6), "frac_of_peak": round(lk["tflops"] / lk["peak"], 4),
            "tile": f"{lk['cfg'].bm}x{lk['cfg'].bn}", "variant": "mfma" if lk["cfg"].variant == 2 else "lds"}
        # (and the unaligned ragged problem, which the heuristic packs into aligned whole tiles)
        for name in ("c1_f32_256", "c2_f32_1024", "k1_f32_long_k", "c5_bf16_ragged", "m8_f16_shard", "m8_f32_shard",
                     "t33_f16_4352x4352x2048"):
            r = time_problem(name, max(5, a.steps // 2), max(2, a.warmup // 2), workspace=True, min_window_ms=5.0, min_warm_ms=20.0)
            out["other_problems"][name]["with_workspace"] = {
                "tflops": round(r["tflops"], 3), "ms_per_step": round(r["ms_per_step"], 6),
                "frac_of_peak": round(r["tflops"] / r["peak"], 4), "split_k": r["cfg"].split_k,
                "packed": r["cfg"].pack == 2, "stream_k_width": r["cfg"].sk_width, "schedule": r["cfg"].schedule,
                "tile": f"{r['cfg'].bm}x{r['cfg'].bn}", "workspace_bytes": r["cfg"].workspace_bytes}
    if fe is not None:
        out["fused_epilogue"] = {"workload": f"{out['config']['workload']} with C = gelu_tanh(A@B + bias) stored "
                                             f"as bf16", "tflops": round(fe["tflops"], 3),
                                 "ms_per_step": round(fe["ms_per_step"], 6),
                                 "frac_of_peak": round(fe["tflops"] / fe["peak"], 4),
                                 "kernel": kernel_name(fe["cfg"], main_res["dtype"])}
    if not a.no_extra and not a.only:
        grouped = {}
        for name in GROUPED:
            r = time_grouped(name, max(5, a.steps // 2), max(2, a.warmup // 2))
            grouped[name] = {"workload": f"{GROUPED[name]['count']} x {GROUPED[name]['M']}x{GROUPED[name]['N']}x"
                                         f"{GROUPED[name]['K']} {GROUPED[name]['dtype']} in one grouped launch",
                             "tflops": round(r["tflops"], 3), "ms_per_step": round(r["ms_per_step"], 6),
                             "frac_of_peak": round(r["tflops"] / r["peak"], 4),
                             "separate_launches_ms": round(r["separate_ms"], 6),
                             "tile": f"{r['cfg'].bm}x{r['cfg'].bn}", "grid": r["cfg"].grid}
        out["grouped"] = grouped
    if a.extended and not a.only:
        # per-launch distribution (median / min) and MALL-cold launches of the two 4096^3 problems
        out["launch_distribution"] = {name: time_distribution(name, n=100 if name.startswith("c4") else 30)
                                      for name in (headline, "c3_f32_4096")}
        out["sclk"] = sclk_under_load(headline)
        for name in ("m8_f16_shard", "m8_f32_shard"):
            if name in out.get("other_problems", {}):
                out["other_problems"][name]["workload"] = ("one GPU's share of the 4096^3 problem split 8 ways by "
                                                           "rows: C=A@B 512x4096x4096 " + name[3:6])
    if not a.no_cpu_baseline and not a.only:
        out["cpu_baseline"] = cpu_baseline(headline, a.cpu_seconds)
        out["cpu_small"] = {"c1_f32_256": cpu_small("c1_f32_256"), "c2_f32_1024": cpu_small("c2_f32_1024", rows=128)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
