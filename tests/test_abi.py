"""CPU tests of the C ABI: the library loads, exports what include/gemm.h declares,
validates arguments before touching a device, and plans launches as documented.

No kernel is launched here: only host-side entry points (gemm_plan, the menu,
status strings) and gemm/gemm_ex calls whose arguments are rejected (or are
empty problems) before any device access.
"""
import ctypes
import os
import re

import pytest

import dense_gemm_06_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(dg.LIB_PATH):
        from dense_gemm_06_amd import build
        build.build()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_symbols_exported():
    names = declared_functions()
    assert set(names) == {"gemm", "gemm_ex", "gemm_plan", "gemm_menu_size", "gemm_menu_entry",
                          "gemm_device_info", "gemm_status_string", "gemm_last_error",
                          "gemm_grouped", "gemm_grouped_plan", "gemm_strided_batched",
                          "gemm_ex_workspace", "gemm_plan_workspace", "gemm_ex_epilogue",
                          "gemm_ex_noalloc"}
    lib = dg.library()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for st in range(6):
        assert dg.gemm_status_string(st).startswith(["GEMM_OK", "GEMM_ERR_INVALID_VALUE", "GEMM_ERR_NULL_POINTER",
                                                     "GEMM_ERR_UNSUPPORTED", "GEMM_ERR_DEVICE",
                                                     "GEMM_ERR_LAUNCH"][st])
    assert dg.gemm_status_string(99) == "unknown gemm_status"


def test_menu_is_complete():
    menu = dg.gemm_menu()
    assert len(menu) == dg.library().gemm_menu_size() == 110
    seen = set()
    for e in menu:
        assert e["lds_bytes"] <= 160 * 1024
        assert e["threads"] in (256, 512)
        seen.add((e["variant"], e["dtype"], e["opb"], e["vec"], e["bm"], e["bn"]))
        if e["variant"] == dg.GEMM_VARIANT_MFMA:
            # one wave grid per workgroup, or two or four that split K (fp32 64 x 64 on
            # either fp32 schedule, 16 x 64 with four groups)
            k_groups = e["threads"] // (e["waves_m"] * e["waves_n"] * 64)
            assert k_groups * e["waves_m"] * e["waves_n"] * 64 == e["threads"] and k_groups in (1, 2, 4)
            assert k_groups == 1 or (e["dtype"] == 0 and (
                ((e["bm"], e["bn"]) == (64, 64) and k_groups == 2 and e["schedule"] in (1, 6, 8)) or
                ((e["bm"], e["bn"]) == (16, 64) and k_groups == 4 and e["schedule"] == 1)))
    for variant in (1, 2):
        for dtype in (0, 1, 2):
            for opb in (0, 1):
                for vec in (0, 1):
                    tiles = {(bm, bn) for (v, d, o, ve, bm, bn) in seen if (v, d, o, ve) == (variant, dtype, opb, vec)}
                    assert len(tiles) >= 2, (variant, dtype, opb, vec)
    assert dg.library().gemm_menu_entry(110, None, None, None, None) == dg.GEMM_ERR_INVALID_VALUE


def plan(M, N, K, dtype="f32", op_b="N", lda=None, ldb=None, ldc=None, a=0, b=0, c=0, cus=256, arch="gfx950",
         req=None):
    lda = lda if lda is not None else max(1, K)
    ldb = ldb if ldb is not None else (max(1, N) if op_b == "N" else max(1, K))
    ldc = ldc if ldc is not None else max(1, N)
    return dg.gemm_plan(0, dg.OP_CODE[op_b], M, N, K, lda, ldb, ldc, dg.DTYPE_CODE[dtype], a, b, c, cus, arch,
                        req, check=False)


def test_plan_benchmark_configs():
    st, c = plan(4096, 4096, 4096, "f16")
    assert st == 0 and c.variant == dg.GEMM_VARIANT_MFMA and (c.bm, c.bn) == (256, 256) and c.grid == 256
    assert c.vec == 1 and c.schedule == 5 and c.threads == 512 and (c.waves_m, c.waves_n) == (2, 4)
    st, c = plan(4096, 4096, 4096, "f32")
    assert st == 0 and c.variant == dg.GEMM_VARIANT_MFMA and c.vec == 1
    # ragged bf16 with column-major B and odd leading dimensions: 16-byte loads from
    # 2-byte-aligned rows on the register-staged software-pipelined kernel, 8 waves
    st, c = plan(3001, 5003, 1037, "bf16", "T", lda=1037, ldb=1037, ldc=5003)
    assert st == 0 and c.variant == dg.GEMM_VARIANT_MFMA and c.vec == 1 and c.schedule == 7
    assert (c.waves_m, c.waves_n) == (2, 4)
    assert (c.bm, c.bn) == (256, 256)
    assert c.tiles_m == -(-3001 // c.bm) and c.tiles_n == -(-5003 // c.bn)


def test_plan_software_pipelined_kernel_where_measured_faster():
    """Schedule 5 with 8 waves for both B layouts; the ping-pong kernel for one round of
    tiles with at most 32 k-tiles; with a fused epilogue, 8 waves for row-major B and
    K of 64 k-tiles or more; the 4-wave form only when asked for."""
    for m, n, k, dt, op_b in ((4096, 4096, 4096, "f16", "N"), (4096, 4096, 4096, "bf16", "N"),
                              (4096, 4096, 2048, "f16", "N"), (8192, 8192, 8192, "f16", "N"),
                              (8192, 8192, 256, "f16", "N"), (8192, 8192, 512, "f16", "N"),
                              (4096, 4096, 4096, "f16", "T"), (4096, 4096, 4096, "bf16", "T"),
                              (8192, 8192, 256, "f16", "T"), (5000, 5000, 5000, "f16", "T")):
        c = plan(m, n, k, dt, op_b)[1]
        assert c.schedule == 5 and (c.waves_m, c.waves_n) == (2, 4), (m, n, k, dt, op_b)
    # one round of 256 tiles and at most 32 k-tiles: the ping-pong kernel
    for k, dt, op_b in ((1024, "f16", "N"), (512, "bf16", "N"), (1024, "bf16", "T")):
        assert plan(4096, 4096, k, dt, op_b)[1].schedule == 2, (k, dt, op_b)
    # the ragged column-major problem: the register-staged form runs it directly, even
    # with a workspace that would allow packing (58 us against 62 packed)
    st, c = dg.gemm_plan_workspace(0, 1, 3001, 5003, 1037, 1037, 1037, 5003, dg.GEMM_BF16, 0x10002, 0x200002,
                                   0x400000, 256, "gfx950", 64 << 20, None)
    assert st == 0 and c.pack == 1 and c.schedule == 7 and c.threads == 512
    # with a fused epilogue: 8 waves from 32 k-tiles on, either B layout; the ping-pong
    # kernel below that
    for op_b, k, sched in ((0, 4096, 5), (1, 4096, 5), (0, 1024, 5), (0, 256, 2), (1, 512, 2)):
        st, c = dg.gemm_plan_workspace(0, op_b, 4096, 4096, k, k, 4096 if op_b == 0 else k, 4096, dg.GEMM_F16, 0, 0,
                                       0, 256, "gfx950", 0, None, epi=dg.epilogue(activation="relu"))
        assert st == 0 and c.schedule == sched and (sched == 2 or c.waves_n == 4), (op_b, k)
    c = plan(4096, 4096, 4096, "f16", req=dg.request(schedule=5, waves_n=2))[1]
    assert c.schedule == 5 and c.threads == 256


def test_plan_ping_pong_eligibility():
    """Whole tiles, K a multiple of 32 and aligned operands, or no ping-pong (edge
    tiles in M and N go to the software-pipelined kernel)."""
    assert plan(4096, 4096, 4096, "bf16")[1].schedule >= 2
    assert plan(4096, 4096, 4096, "f16", "T")[1].schedule >= 2
    assert plan(4096, 4096, 4096 + 16, "f16")[1].schedule == 5   # the software-pipelined kernel's K tail
    for sched in (2, 4):
        st, _ = plan(4096, 4096, 4096 + 16, "f16", req=dg.request(schedule=sched))
        assert st == dg.GEMM_ERR_UNSUPPORTED
    assert plan(4096 + 8, 4096, 4096, "f16")[1].schedule == 5
    for sched in (2, 4):
        # edge tiles in M and N: yes; row-major B with N not a multiple of 8: no
        assert plan(4096 + 8, 4096, 4096, "f16", req=dg.request(schedule=sched))[0] == 0
        st, _ = plan(4096, 4001, 4096, "f16", ldb=4008, req=dg.request(schedule=sched))
        assert st == dg.GEMM_ERR_UNSUPPORTED
    assert plan(4096, 4096, 4096, "f16", a=2)[1].schedule == 7    # A not 16-byte aligned
    assert plan(4096, 4096, 4096, "f32")[1].schedule not in (2, 3, 4, 5, 7)
    st, _ = plan(4096, 4096, 4000 + 8, "f16", req=dg.request(schedule=2))   # K not a multiple of 32
    assert st == dg.GEMM_ERR_UNSUPPORTED


def test_plan_software_pipelined_edge_tiles():
    """Schedule 5 takes M and N that are not multiples of 256 (row-major B only with N a
    multiple of 8); K must stay a multiple of 32 and the operands 16-byte aligned."""
    for op_b, sched in (("N", 5), ("T", 5)):
        st, c = plan(4000, 4000, 4000, "f16", op_b)
        assert st == 0 and c.schedule == sched and (c.tiles_m, c.tiles_n) == (16, 16), op_b
    st, c = plan(4000, 4001, 4096, "f16", "N", ldb=4008)     # a 16-byte chunk would straddle N
    assert st == 0 and c.schedule == 7
    st, _ = plan(4000, 4001, 4096, "f16", "N", ldb=4008, req=dg.request(schedule=5))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    st, c = plan(4000, 4001, 4096, "f16", "T")
    assert st == 0 and c.schedule in (2, 5)
    assert plan(4000, 4000, 4000 + 8, "f16")[1].schedule == 5   # a partial last k-tile
    st, c = plan(4000, 4000, 4004, "f16", lda=4008)             # K not a multiple of 8
    assert st == 0 and c.schedule == 7
    assert plan(4000, 4000, 4000, "f16", lda=4004)[1].schedule == 7   # rows not 16-byte aligned


def test_plan_three_stage_fp32():
    """Schedule 6 (fp32 256 x 128, three LDS stages) where the grid fills the machine
    and the direct-copy tiles do not apply (K not a multiple of 32, or rows not 16-byte
    aligned), either B layout, and its 64 x 64 form for one round of tiles; never for
    16-bit inputs, never split."""
    for op_b in "NT":
        for shape, lda in (((4000, 4096, 3001), None), ((4096, 4096, 4096), 4097), ((8192, 8192, 8192), 8194)):
            st, c = plan(*shape, "f32", op_b, lda=lda)
            assert st == 0 and c.schedule == 6 and (c.bm, c.bn) == (256, 128) and c.threads == 512, (shape, op_b)
    # one round of 64 x 64 tiles on unaligned rows: the same schedule with two K
    # groups on that tile
    st, c = plan(1024, 1024, 1024, "f32", lda=1025)
    assert st == 0 and c.schedule == 6 and (c.bm, c.bn) == (64, 64)
    # short K: the large tiles' fixed cost per round of tiles outweighs their faster
    # k loop; two resident 128 x 128 register-staged tiles per CU
    for shape in ((8192, 8192, 256), (8192, 8192, 512), (12288, 12288, 512)):
        st, c = plan(*shape, "f32")
        assert st == 0 and c.schedule == 1 and (c.bm, c.bn) == (128, 128), shape
    # few tiles of long K split on the 64 x 64 direct-copy tile (512^2 x 8192: 46 us
    # split four ways, against 57 on the register-staged tile)
    st, c = wplan(512, 512, 8192, "f32")
    assert st == 0 and c.schedule == 8 and c.split_k > 1
    # forced, with a K split: refused (schedule 6 has no sliced form)
    st, _ = wplan(4096, 4096, 4096, "f32", req=dg.request(schedule=6, split_k=2), check=False)
    assert st != 0
    st, _ = plan(4096, 4096, 4096, "f16", req=dg.request(schedule=6))
    assert st == dg.GEMM_ERR_UNSUPPORTED


def test_plan_never_selects_removed_schedule():
    """Schedule 3 (a kernel that faulted on the device) was removed: no menu entry has it,
    it is never chosen, and a forced request is refused."""
    assert all(e["schedule"] != 3 for e in dg.gemm_menu())
    for dtype in ("f16", "bf16"):
        for op_b in "NT":
            for shape in ((4096, 4096, 4096), (256, 512, 32), (8192, 8192, 8192)):
                st, c = plan(*shape, dtype, op_b)
                assert st == 0 and c.schedule != 3
            st, _ = plan(4096, 4096, 4096, dtype, op_b, req=dg.request(schedule=3))
            assert st == dg.GEMM_ERR_UNSUPPORTED
    assert "removed" in dg.gemm_last_error()


def test_plan_persistent_grid():
    """max_grid below the tile count on a single call: the persistent form of the
    8-wave schedule-5 kernel (whole k-tiles of 32, at least four, no split); a cap at
    or above the tile count changes nothing; shapes the persistent form cannot take
    are refused with the reason."""
    for dtype in ("f16", "bf16"):
        for op_b in "NT":
            st, c = plan(8192, 8192, 1024, dtype, op_b, req=dg.request(max_grid=256))
            assert st == 0 and c.grid == 256 and c.schedule == 5 and c.threads == 512 and c.max_grid == 256
            assert c.tiles_m * c.tiles_n == 1024 and c.xcd_remap == 1
            st, c = plan(1000, 1304, 256, dtype, op_b, req=dg.request(max_grid=3))
            assert st == 0 and c.grid == 3 and c.schedule == 5 and c.xcd_remap == 0
    # without a cap: the persistent grid of one workgroup per compute unit where the
    # tiles outnumber the compute units, one workgroup per tile otherwise
    for dtype, op_b in (("f16", "N"), ("bf16", "T")):
        st, c = plan(8192, 8192, 1024, dtype, op_b)
        assert st == 0 and c.schedule == 5 and c.threads == 512 and c.grid == 256 and c.xcd_remap == 1
        st, c = plan(8192, 8192, 1024, dtype, op_b, cus=304)
        assert st == 0 and c.schedule == 5 and c.grid == 304
        st, c = plan(8192, 8192, 1024, dtype, op_b, req=dg.request(max_grid=1 << 20))
        assert st == 0 and c.grid == 1024
    st, c = plan(8192, 8192, 1000, "f16")   # partial last k-tile: no persistent form
    assert st == 0 and c.grid == c.tiles_m * c.tiles_n
    st, c = plan(4096, 4096, 4096, "f16", req=dg.request(max_grid=256))
    assert st == 0 and c.grid == 256 and c.schedule == 5
    st, c = plan(4096, 4096, 4096, "f16", req=dg.request(max_grid=100000))
    assert st == 0 and c.grid == 256
    # the persistent form needs at least four whole k-tiles of 32
    for K in (96, 1000, 1036):
        st, c = plan(8192, 8192, K, "f16", req=dg.request(max_grid=256))
        assert st == dg.GEMM_ERR_UNSUPPORTED and "max_grid" in dg.gemm_last_error(), K
    # the 4-wave form, a split and the other schedules have no persistent single-call form
    st, c = plan(8192, 8192, 1024, "f16", req=dg.request(max_grid=256, waves_n=2, schedule=5))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    st, c = plan(8192, 8192, 1024, "f16", req=dg.request(max_grid=256, schedule=7))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    st, c = plan(8192, 8192, 1024, "f32", req=dg.request(max_grid=256))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    st, c = plan(512, 512, 1024, "f32", req=dg.request(max_grid=256))
    assert st == 0 and c.grid <= 256
    st, c = plan(64, 64, 64, "f16", req=dg.request(max_grid=-1))
    assert st == dg.GEMM_ERR_INVALID_VALUE


def test_plan_cache_returns_the_uncached_plan():
    """The planner keeps successful plans in a cache keyed on everything a plan
    depends on. Repeated and interleaved calls must give what a first call gives:
    same problem twice, then the alignment class, a request field, the workspace and
    the CU count changed one at a time (each changes the plan here), and a failing
    call between them (failures are not cached and keep their message)."""
    fields = [f for f, _ in dg.gemm_config._fields_ if f != "est_cycles"]

    def snap(c):
        return tuple(getattr(c, f) for f in fields)

    cases = [
        dict(M=3001, N=5003, K=1037, dtype="bf16", op_b="T", a=0, b=0),        # aligned bases, odd lds
        dict(M=3001, N=5003, K=1037, dtype="bf16", op_b="T", a=1, b=1),        # not element-aligned
        dict(M=4096, N=4096, K=4096, dtype="f16", op_b="N", a=0, b=0),
        dict(M=4096, N=4096, K=4096, dtype="f16", op_b="N", a=8, b=0),         # not 16-byte aligned
        dict(M=8192, N=8192, K=1024, dtype="f16", op_b="N", a=0, b=0),         # persistent grid
        dict(M=8192, N=8192, K=1024, dtype="f16", op_b="N", a=0, b=0, cus=128),
        dict(M=4096, N=4096, K=4096, dtype="f16", op_b="N", a=0, b=0, req=dict(schedule=2)),
        dict(M=4096, N=4096, K=4096, dtype="f16", op_b="N", a=0, b=0, req=dict(waves_n=2)),
        dict(M=256, N=256, K=16384, dtype="f32", op_b="N", a=0, b=0),
    ]

    def run(cs):
        kw = dict(cs)
        req = kw.pop("req", None)
        cus = kw.pop("cus", 256)
        st, c = plan(kw["M"], kw["N"], kw["K"], kw["dtype"], kw["op_b"], a=kw["a"], b=kw["b"], cus=cus,
                     req=dg.request(**req) if req else None)
        assert st == 0
        return snap(c)

    first = [run(cs) for cs in cases]
    assert len(set(first)) == len(first), "each case changes the plan"
    for _ in range(3):
        for i, cs in enumerate(cases):
            assert run(cs) == first[i]
            st, _ = plan(4096, 4096, 4096, "f16", req=dg.request(schedule=3))
            assert st == dg.GEMM_ERR_UNSUPPORTED and "removed" in dg.gemm_last_error()
    # workspace: split K appears only with one (gemm_plan_workspace)
    st, c0 = dg.gemm_plan_workspace(0, 0, 256, 256, 16384, 16384, 256, 256, dg.GEMM_F32, 0, 0, 1 << 40, 256,
                                    "gfx950", 0, None, check=False)
    st1, c1 = dg.gemm_plan_workspace(0, 0, 256, 256, 16384, 16384, 256, 256, dg.GEMM_F32, 0, 0, 1 << 40, 256,
                                     "gfx950", 1 << 26, None, check=False)
    st2, c2 = dg.gemm_plan_workspace(0, 0, 256, 256, 16384, 16384, 256, 256, dg.GEMM_F32, 0, 0, 1 << 40, 256,
                                     "gfx950", 0, None, check=False)
    assert st == st1 == st2 == 0 and c0.split_k == 1 and c1.split_k > 1 and snap(c2) == snap(c0)


def test_plan_fp32_choices_follow_measurements():
    """fp32 tile choices (no workspace) on shapes where the pick measured fastest by at
    least 3% against every other tile family (medians of five passes in shuffled
    order, one box; us, the pick against the next best): the direct-copy 64 x 64 tile
    for one to a few rounds of its tiles, the direct-copy 128 x 128 tile for one round
    of long K and for column-major B, the 256 x 128 one for row-major B at 4096^3,
    five resident 64 x 64 register-staged tiles for many tiles of short K, two
    resident 128 x 128 ones for K = 256, 16 x 64 tiles for few tiles."""
    cases = {  # (M, N, K, B layout): (schedule, bm, threads)
        (1024, 1024, 1024, "N"): (8, 64, 512),     # 22.1 against 25.0
        (1024, 1024, 1024, "T"): (8, 64, 512),     # 21.7 against 24.3
        (1024, 1024, 4096, "T"): (8, 64, 512),     # 72.8 against 85.0
        (1024, 1024, 16384, "N"): (8, 64, 512),    # 272 against 329
        (768, 768, 4096, "N"): (8, 64, 512),       # 71.1 against 83.0
        (2048, 2048, 2048, "N"): (9, 128, 512),    # 135.8 against 147.6
        (2048, 2048, 2048, "T"): (9, 128, 512),    # 129.0 against 145.7
        (2048, 2048, 8192, "T"): (9, 128, 512),    # 503 against 548
        (1024, 4096, 1024, "T"): (9, 128, 512),    # 69.7 against 76.5
        (4096, 4096, 4096, "T"): (9, 128, 512),    # 990 against 1022
        (4096, 4096, 4096, "N"): (9, 256, 512),    # 1010-1017 against 1031-1040 (128 x 128)
        (3072, 3072, 1024, "N"): (1, 64, 256),     # 166.8 against 175.3
        (3072, 3072, 1024, "T"): (1, 64, 256),     # 167.6 against 176.0
        (1536, 6144, 1024, "N"): (1, 64, 256),     # 166.1 against 175.4
        (8192, 8192, 256, "T"): (1, 128, 256),     # 294.5 against 306.5
        (512, 512, 2048, "N"): (1, 16, 256),       # 22.8 against 36.5
        (640, 640, 16384, "N"): (1, 16, 256),      # 206.7 against 267.8
        (256, 2048, 8192, "N"): (1, 16, 256),      # 106.8 against 137.6
    }
    for (M, N, K, op_b), want in cases.items():
        st, c = plan(M, N, K, "f32", op_b)
        assert st == 0 and (c.schedule, c.bm, c.threads) == want, ((M, N, K, op_b), c.schedule, c.bm, c.threads)
    # a partial tile in M or N slows the register-staged tiles' k loop (the edge tile
    # sets the launch's time), not the direct-copy tiles' clamped copies: 1024 x 1028 x
    # 4096 on the direct-copy 64 x 64 tile 146.6 us against 228 on 64 x 64
    # register-staged tiles (1024 x 1088: 146.6 against 160)
    st, c = plan(1024, 1028, 4096, "f32")
    assert st == 0 and c.schedule == 8


def test_plan_stream_k():
    """The stream-K tail of the persistent software-pipelined kernel: chosen with a
    workspace where it was timed faster (a tail of 33 or 32 tiles behind whole rounds),
    not where it was timed slower (a tail of 68 or 144 tiles) or where a round is
    exactly full; never without a workspace or with stream_k = 1; forced with
    stream_k = 2 where it applies and refused with the reason where it does not."""
    def wsplan(M, N, K, dt, op_b=0, ws=1 << 30, req=None):
        return dg.gemm_plan_workspace(0, op_b, M, N, K, K, N if op_b == 0 else K, N, dg.DTYPE_CODE[dt], 4096, 4096,
                                      4096, 256, "gfx950", ws, req, check=False)
    for (M, N, K, dt, op_b) in ((4352, 4352, 2048, "f16", 0), (4352, 4352, 8192, "f16", 0),
                                (4352, 4352, 4096, "bf16", 1), (8448, 8192, 2048, "f16", 0)):
        st, c = wsplan(M, N, K, dt, op_b)
        tail = c.tiles_total % c.grid
        assert st == 0 and c.stream_k == 2 and c.schedule == 5 and c.threads == 512 and c.grid == 256, (M, N, K)
        assert tail in (32, 33) and c.sk_width > tail and c.launches == 2 and c.split_k == 1
        assert c.workspace_bytes == c.sk_width * 512 * 1024
        st, c1 = wsplan(M, N, K, dt, op_b, req=dg.request(stream_k=1))
        assert st == 0 and c1.stream_k == 1 and c1.sk_width == 0 and c1.launches == 1 and c1.workspace_bytes == 0
        st, c0 = wsplan(M, N, K, dt, op_b, ws=0)
        assert st == 0 and c0.stream_k == 1 and c0.workspace_bytes == 0
        # a workspace below the chosen width's need: a narrower width or none
        st, cs = wsplan(M, N, K, dt, op_b, ws=c.workspace_bytes - 1)
        assert st == 0 and (cs.stream_k == 1 or cs.sk_width < c.sk_width)
    for (M, N, K) in ((4608, 4608, 1024), (5120, 5120, 4096), (4096, 4096, 4096), (8192, 8192, 2048)):
        st, c = wsplan(M, N, K, "f16")
        assert st == 0 and c.stream_k == 1, (M, N, K)
    # forced: the width asked for, the grid of a max_grid, fewer tiles than the grid
    st, c = wsplan(768, 1024, 512, "f16", req=dg.request(stream_k=2, max_grid=8, sk_width=5))
    assert st == 0 and c.stream_k == 2 and c.grid == 8 and c.sk_width == 5 and c.tiles_total == 12
    st, c = wsplan(512, 512, 2048, "bf16", op_b=1, req=dg.request(stream_k=2))
    assert st == 0 and c.stream_k == 2 and c.grid == 256 and c.tiles_total == 4 and 4 < c.sk_width <= 64
    # refused: a round exactly full, too few k-tiles, fp32, a width not above the tail,
    # shares under 4 k-tiles, too little workspace, a split asked for as well
    bad = [((4096, 4096, 4096, "f16", 0), dg.request(stream_k=2)),
           ((4352, 4352, 224, "f16", 0), dg.request(stream_k=2)),
           ((4352, 4352, 2048, "f32", 0), dg.request(stream_k=2)),
           ((4352, 4352, 2048, "f16", 0), dg.request(stream_k=2, sk_width=33)),
           ((4352, 4352, 256, "f16", 0), dg.request(stream_k=2, sk_width=256)),
           ((4352, 4352, 2048, "f16", 0), dg.request(stream_k=2, split_k=2))]
    for (M, N, K, dt, op_b), req in bad:
        st, _ = wsplan(M, N, K, dt, op_b, req=req)
        assert st == dg.GEMM_ERR_INVALID_VALUE and "stream_k" in dg.gemm_last_error(), (M, N, K, dt)
    st, _ = wsplan(4352, 4352, 2048, "f16", ws=1 << 20, req=dg.request(stream_k=2))
    assert st == dg.GEMM_ERR_INVALID_VALUE and "workspace" in dg.gemm_last_error()
    for req in (dg.request(stream_k=3), dg.request(stream_k=-1), dg.request(sk_width=-2)):
        st, _ = wsplan(4352, 4352, 2048, "f16", req=req)
        assert st == dg.GEMM_ERR_INVALID_VALUE


def test_plan_16bit_choices_follow_measurements():
    """16-bit choices with a workspace on shapes where the choice was timed against the
    previous model's (medians of five alternated passes, one box): few tiles facing a
    long K split on the 256 x 256 software-pipelined kernel or on smaller register-staged
    tiles, which the previous model left unsplit on 64 x 64 or 128 x 128 tiles."""
    cases = {  # (M, N, K), dtype, opB: (schedule, bm, split)   time against the previous choice
        ((768, 1024, 16384), "f16", 0): (5, 256, 16),   # 46.0 us against 129.7
        ((1536, 1536, 8192), "f16", 0): (5, 256, 6),    # 54.7 against 102.3 (four slices 54.2, within noise)
        ((512, 3072, 8192), "bf16", 1): (5, 256, 8),    # 42.6 against 68.5 (six slices 43.6)
        ((2048, 3072, 16384), "bf16", 1): (5, 256, 2),  # 188.3 against 280.6
        ((768, 1024, 8192), "f16", 0): (1, 128, 8),     # 32.2 against 66.1
        ((512, 768, 4096), "f16", 0): (1, 64, 4),       # 16.6 against 33.8
    }
    for ((M, N, K), dt, op_b), want in cases.items():
        st, c = dg.gemm_plan_workspace(0, op_b, M, N, K, K, N if op_b == 0 else K, N, dg.DTYPE_CODE[dt], 4096, 4096,
                                       4096, 256, "gfx950", 1 << 30, None)
        assert st == 0 and (c.schedule, c.bm, c.split_k) == want, ((M, N, K), dt, c.schedule, c.bm, c.split_k)
        assert c.grid == c.tiles_total and c.workspace_bytes == c.split_k * M * ((N + 3) // 4 * 4) * 4
    # without a workspace nothing splits, and the same problems keep one launch
    st, c = dg.gemm_plan_workspace(0, 0, 768, 1024, 16384, 16384, 1024, 1024, dg.GEMM_F16, 4096, 4096, 4096, 256,
                                   "gfx950", 0, None)
    assert st == 0 and c.split_k == 1 and c.launches == 1


def test_plan_fills_the_machine():
    """A smaller problem gets smaller tiles so that the grid covers the compute units."""
    st, c = plan(1024, 1024, 1024, "f32")
    assert st == 0 and c.grid >= 256
    # 256^3: the 16 x 64 tile with K over four wave groups (64 workgroups; 64 x 64
    # tiles would give 16)
    for op_b in "NT":
        st, c = plan(256, 256, 256, "f32", op_b)
        assert st == 0 and (c.bm, c.bn) == (16, 64) and c.grid == 64 and c.threads == 256
    st, c = plan(512, 512, 512, "f32")
    assert st == 0 and (c.bm, c.bn) == (16, 64) and c.grid == 256
    # 1024^3: 64 x 64 tiles fill the machine; one round of them on the direct-copy
    # tile with two K groups (schedule 8), or on the three-stage schedule where the
    # operands are not 16-byte aligned
    for op_b in "NT":
        st, c = plan(1024, 1024, 1024, "f32", op_b)
        assert st == 0 and (c.bm, c.bn) == (64, 64) and c.schedule == 8 and c.threads == 512 and c.grid == 256
    st, c = plan(1024, 1024, 1024, "f32", lda=1025)
    assert st == 0 and (c.bm, c.bn) == (64, 64) and c.schedule == 6
    st, c = plan(1024, 1024, 1000, "f32")   # K not a multiple of 64
    assert st == 0 and c.schedule != 8
    st, c = plan(2048, 2048, 2048, "f32")
    assert st == 0 and c.schedule != 6 or c.bm == 256
    # a tall-skinny problem still picks a tile count close to the CU count or more
    st, c = plan(8192, 64, 4096, "f16")
    assert st == 0 and c.grid >= 64


def test_plan_alignment_rules():
    # element-aligned bases: 16-byte loads, whatever the row alignment
    assert plan(512, 512, 512, "f16", a=2)[1].vec == 1
    assert plan(512, 512, 512, "f16", lda=516)[1].vec == 1     # 1032 bytes per row
    assert plan(512, 512, 512, "f16", lda=520)[1].vec == 1     # 1040 bytes = 65 x 16
    assert plan(512, 512, 512, "f32", ldb=514)[1].vec == 1
    # a base not aligned to the element: element-wise loads
    assert plan(512, 512, 512, "f16", a=1)[1].vec == 0
    assert plan(512, 512, 512, "f32", b=6)[1].vec == 0
    # the direct global -> LDS copies of the whole-tile kernels need 16-byte rows
    assert plan(4096, 4096, 4096, "f16")[1].schedule == 5
    # (otherwise the register-staged form of the software-pipelined kernel runs)
    for kw in (dict(a=2), dict(lda=4100), dict(b=8), dict(ldb=4100)):
        st, c = plan(4096, 4096, 4096, "f16", **kw)
        assert st == 0 and c.schedule == 7 and c.vec == 1, kw
        st, _ = plan(4096, 4096, 4096, "f16", req=dg.request(schedule=5), **kw)
        assert st == dg.GEMM_ERR_UNSUPPORTED, kw
    # forcing 16-byte loads on bases not aligned to the element is refused
    st, _ = plan(512, 512, 512, "f16", a=1, req=dg.request(vec=1))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    assert plan(512, 512, 512, "f16", a=2, req=dg.request(vec=1))[0] == 0


def test_plan_forced_configurations():
    st, c = plan(1000, 1000, 1000, "f32", req=dg.request(variant=dg.GEMM_VARIANT_LDS))
    assert st == 0 and c.variant == dg.GEMM_VARIANT_LDS and c.thread_m in (4, 8)
    st, c = plan(1000, 1000, 1000, "f16", req=dg.request(variant=dg.GEMM_VARIANT_MFMA, bm=128, bn=128))
    assert st == 0 and (c.bm, c.bn) == (128, 128)
    st, c = plan(1000, 1000, 1000, "f16", req=dg.request(bm=96))
    assert st == dg.GEMM_ERR_UNSUPPORTED and "no compiled kernel" in dg.gemm_last_error()
    st, c = plan(1000, 1000, 1000, "f16", req=dg.request(xcd_remap=0, group_m=3))
    assert st == 0 and c.xcd_remap == 0 and c.group_m == 3
    st, _ = plan(1000, 1000, 1000, "f16", req=dg.request(variant=7))
    assert st == dg.GEMM_ERR_INVALID_VALUE


@pytest.mark.parametrize("args,status,needle", [
    (dict(M=-1, N=4, K=4), dg.GEMM_ERR_INVALID_VALUE, "negative size"),
    (dict(M=4, N=4, K=4, lda=3), dg.GEMM_ERR_INVALID_VALUE, "lda"),
    (dict(M=4, N=4, K=4, ldb=3), dg.GEMM_ERR_INVALID_VALUE, "ldb"),
    (dict(M=4, N=4, K=8, op_b="T", ldb=7), dg.GEMM_ERR_INVALID_VALUE, "column-major"),
    (dict(M=4, N=4, K=4, ldc=3), dg.GEMM_ERR_INVALID_VALUE, "ldc"),
    (dict(M=4, N=4, K=4, ldc=1 << 61), dg.GEMM_ERR_INVALID_VALUE, "extent"),
    (dict(M=1 << 29, N=4, K=4, ldc=(1 << 62) // (1 << 29)), dg.GEMM_ERR_INVALID_VALUE, "extent"),
    (dict(M=4, N=4, K=4, ldc=(1 << 63) - 1), dg.GEMM_ERR_INVALID_VALUE, "extent"),
    (dict(M=4, N=4, K=4, arch="gfx942"), dg.GEMM_ERR_DEVICE, "gfx942"),
    (dict(M=4, N=4, K=4, cus=0), dg.GEMM_ERR_INVALID_VALUE, "compute-unit"),
    (dict(M=1 << 30, N=4, K=4), dg.GEMM_ERR_UNSUPPORTED, "2^30"),
    (dict(M=4, N=4, K=4, lda=1 << 23), dg.GEMM_ERR_UNSUPPORTED, "2^23"),
])
def test_plan_rejections(args, status, needle):
    st, _ = plan(**args)
    assert st == status
    assert needle in dg.gemm_last_error()


def test_plan_bad_enums():
    lib = dg.library()
    out = dg.gemm_config()
    assert lib.gemm_plan(0, 0, 4, 4, 4, 4, 4, 4, 3, 0, 0, 0, 256, b"gfx950", None, ctypes.byref(out)) == 1
    assert lib.gemm_plan(0, 2, 4, 4, 4, 4, 4, 4, 0, 0, 0, 0, 256, b"gfx950", None, ctypes.byref(out)) == 1
    assert lib.gemm_plan(1, 0, 4, 4, 4, 4, 4, 4, 0, 0, 0, 0, 256, b"gfx950", None, ctypes.byref(out)) == 3
    assert "opA" in dg.gemm_last_error()
    assert lib.gemm_plan(0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 0, 0, 256, None, None, ctypes.byref(out)) == 4
    assert lib.gemm_plan(0, 0, 4, 4, 4, 4, 4, 4, 0, 0, 0, 0, 256, b"gfx950", None, None) == 2


def test_gemm_rejects_before_device_access():
    """Invalid arguments are refused before any HIP call (works without a GPU)."""
    f32 = dg.GEMM_F32
    assert dg.gemm(4, 4, 4, 0x1000, 4, 0x2000, 4, 0, 4, f32, check=False) == dg.GEMM_ERR_NULL_POINTER
    assert dg.gemm(4, 4, 4, 0, 4, 0x2000, 4, 0x3000, 4, f32, check=False) == dg.GEMM_ERR_NULL_POINTER
    assert dg.gemm(-4, 4, 4, 0x1000, 4, 0x2000, 4, 0x3000, 4, f32, check=False) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm(4, 4, 4, 0x1000, 4, 0x2000, 4, 0x3000, 4, 9, check=False) == dg.GEMM_ERR_INVALID_VALUE
    # C overlapping A (A spans 64 bytes from 0x1000; C starts inside it)
    assert dg.gemm(4, 4, 4, 0x1000, 4, 0x8000, 4, 0x1020, 4, f32, check=False) == dg.GEMM_ERR_INVALID_VALUE
    assert "overlaps" in dg.gemm_last_error()
    # C overlapping column-major B
    assert dg.gemm_ex(0, 1, 4, 4, 4, 0x1000, 4, 0x8000, 4, 0x8010, 4, f32, check=False) == \
        dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_ex(1, 0, 4, 4, 4, 0x1000, 4, 0x8000, 4, 0x9000, 4, f32, check=False) == dg.GEMM_ERR_UNSUPPORTED
    # empty products succeed without a launch; NULL pointers are fine when nothing is touched
    assert dg.gemm(0, 4, 4, 0, 4, 0, 4, 0, 4, f32, check=False) == dg.GEMM_OK
    assert dg.gemm(4, 0, 4, 0, 4, 0, 4, 0, 1, f32, check=False) == dg.GEMM_OK
    assert dg.gemm_last_error() == ""
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm(4, 4, 4, 0, 4, 0x2000, 4, 0x3000, 4, f32)
    assert ei.value.status == dg.GEMM_ERR_NULL_POINTER and "NULL operand" in str(ei.value)


# ----------------------------------------------------------------------------- grouped calls
def gp(M, N, K, a=1 << 20, b=1 << 24, c=1 << 28, lda=None, ldb=None, ldc=None, batch=1, sa=0, sb=0, sc=0,
       op_b="N"):
    lda = lda if lda is not None else max(1, K)
    ldb = ldb if ldb is not None else (max(1, N) if op_b == "N" else max(1, K))
    ldc = ldc if ldc is not None else max(1, N)
    return dg.problem(M, N, K, a, lda, b, ldb, c, ldc, batch=batch, stride_a=sa, stride_b=sb, stride_c=sc)


def distinct(shapes, dtype_size=4):
    """Problems at far-apart fake addresses (planning uses addresses for alignment only)."""
    return [gp(M, N, K, a=(i + 1) << 32, b=(i + 1) << 33, c=(i + 1) << 34) for i, (M, N, K) in enumerate(shapes)]


def test_grouped_plan_counts_tiles_and_launches():
    probs = distinct([(256, 256, 256)] * 4)
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, probs)
    assert st == 0 and c.schedule == 1 and c.launches == 1
    assert c.tiles_total == 4 * c.tiles_m * c.tiles_n and 0 < c.grid <= c.tiles_total
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F16, distinct([(100, 90, 80)] * 33))
    assert st == 0 and c.launches == 3
    # empty problems take no segment and no tile
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F16, distinct([(0, 90, 80), (100, 0, 80), (100, 90, 80)]))
    assert st == 0 and c.launches == 1 and c.tiles_total == c.tiles_m * c.tiles_n
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F16, [])
    assert st == 0 and c.launches == 0 and c.tiles_total == 0


def test_grouped_plan_schedules():
    """Grouped calls run the register-staged schedule (1) or, where every problem is
    16-byte aligned with K a multiple of 32 and at least 128 (row-major B: N a multiple
    of 8), the persistent software-pipelined kernel (schedule 5, 8 waves); never the
    other whole-tile schedules."""
    for dt in (dg.GEMM_F16, dg.GEMM_BF16):
        for op_b in "NT":
            st, c = dg.gemm_grouped_plan(0, dg.OP_CODE[op_b], dt, [gp(4096, 4096, 1024, op_b=op_b)] * 1 +
                                         [gp(2048, 1000, 512, a=1 << 36, b=1 << 37, c=1 << 38, op_b=op_b)])
            assert st == 0 and c.schedule == 5 and c.threads == 512 and c.grid == 256 and c.xcd_remap == 1
        # a batch at 16-byte strides keeps it; an odd stride, K not a multiple of 32,
        # K below 128, N not a multiple of 8 for row-major B, or fp32 do not
        # (16 members of 16 tiles: enough 256 x 256 tiles to fill the machine)
        ok = gp(1024, 1024, 256, batch=16, sa=1024 * 256 + 8, sb=256 * 1024 + 8, sc=1024 * 1024)
        assert dg.gemm_grouped_plan(0, 0, dt, [ok])[1].schedule == 5
        for bad in (gp(1024, 1024, 256, batch=16, sa=1024 * 256 + 1, sb=256 * 1024, sc=1024 * 1024),
                    gp(4096, 4096, 1000), gp(4096, 4096, 96), gp(4096, 4092, 256),
                    gp(4096, 4096, 256, a=(1 << 20) + 2)):
            st, c = dg.gemm_grouped_plan(0, 0, dt, [bad])
            assert st == 0 and c.schedule == 1, bad
            st, _ = dg.gemm_grouped_plan(0, 0, dt, [bad], req=dg.request(schedule=5), check=False)
            assert st == dg.GEMM_ERR_UNSUPPORTED
        for sched in (2, 4, 6, 7):
            st, _ = dg.gemm_grouped_plan(0, 0, dt, distinct([(4096, 4096, 4096)]), req=dg.request(schedule=sched),
                                         check=False)
            assert st == dg.GEMM_ERR_UNSUPPORTED
        st, c = dg.gemm_grouped_plan(0, 0, dt, distinct([(4096, 4096, 4096)]), req=dg.request(schedule=1))
        assert st == 0 and c.schedule == 1
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, distinct([(4096, 4096, 4096)]))
    assert st == 0 and c.schedule == 1


def test_grouped_plan_max_grid_and_vec():
    probs = distinct([(512, 512, 64)] * 4)
    st, c = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, probs, req=dg.request(max_grid=5))
    assert st == 0 and c.grid == 5
    assert dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, probs)[1].vec == 1
    # batch strides are in elements: an odd one keeps the 16-byte path
    odd = probs + [gp(64, 64, 64, a=1 << 40, b=1 << 41, c=1 << 42, batch=2, sa=64 * 64 + 1, sb=4096, sc=4096)]
    assert dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, odd)[1].vec == 1
    # one base not aligned to the element turns it off for the whole call
    bad = probs + [gp(64, 64, 64, a=(1 << 40) + 2, b=1 << 41, c=1 << 42)]
    assert dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, bad)[1].vec == 0
    st, _ = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, bad, req=dg.request(vec=1), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("bad,status", [
    (dict(M=-1), dg.GEMM_ERR_INVALID_VALUE),
    (dict(lda=3), dg.GEMM_ERR_INVALID_VALUE),          # lda < K
    (dict(batch=-2), dg.GEMM_ERR_INVALID_VALUE),
    (dict(sa=-1), dg.GEMM_ERR_INVALID_VALUE),
    (dict(batch=2, sc=10), dg.GEMM_ERR_INVALID_VALUE),  # batch outputs would overlap
    (dict(ldc=1 << 31), dg.GEMM_ERR_UNSUPPORTED),
])
def test_grouped_validation(bad, status):
    kw = dict(M=16, N=16, K=16)
    kw.update(bad)
    probs = [gp(16, 16, 16)] + [gp(**kw, a=1 << 36, b=1 << 37, c=1 << 38)]
    st, _ = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, probs, check=False)
    assert st == status
    assert "problem 1" in dg.gemm_last_error()
    # the device entry point rejects the same arguments before touching any device
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, probs, check=False) == status


def test_grouped_rejects_without_device_access():
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, [], check=False) == dg.GEMM_OK
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, None, count=2, check=False) == dg.GEMM_ERR_NULL_POINTER
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, [gp(4, 4, 4)], count=-1, check=False) == dg.GEMM_ERR_INVALID_VALUE
    # a problem without output elements is a no-op even with NULL operands
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, [gp(0, 4, 4, a=0, b=0, c=0)], check=False) == dg.GEMM_OK
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, [gp(4, 4, 4, c=0)], check=False) == dg.GEMM_ERR_NULL_POINTER
    # K = 0 needs no inputs
    two = [gp(4, 4, 4), gp(4, 4, 0, a=0, b=0, c=0)]
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, two, check=False) == dg.GEMM_ERR_NULL_POINTER


@pytest.mark.parametrize("case", ["c_over_own_a", "c_over_other_b", "outputs_overlap", "batch_reaches_input"])
def test_grouped_rejects_overlaps(case):
    base = 1 << 30
    p0 = gp(64, 64, 64, a=base, b=base + (1 << 20), c=base + (2 << 20))
    if case == "c_over_own_a":
        p0 = gp(64, 64, 64, a=base, b=base + (1 << 20), c=base + 64)
        probs = [p0]
    elif case == "c_over_other_b":
        probs = [p0, gp(64, 64, 64, a=base + (3 << 20), b=base + (4 << 20), c=base + (1 << 20) + 128)]
    elif case == "outputs_overlap":
        probs = [p0, gp(64, 64, 64, a=base + (3 << 20), b=base + (4 << 20), c=base + (2 << 20) + 256)]
    else:
        # the last output of a batch reaches into the next problem's A
        probs = [gp(64, 64, 64, a=base, b=base + (1 << 20), c=base + (2 << 20), batch=4, sc=1 << 18),
                 gp(64, 64, 64, a=base + (2 << 20) + 3 * (1 << 18) * 4 + 100, b=base + (5 << 20), c=base + (6 << 20))]
    assert dg.gemm_grouped(0, 0, dg.GEMM_F32, probs, check=False) == dg.GEMM_ERR_INVALID_VALUE
    assert "overlap" in dg.gemm_last_error()


def test_strided_batched_is_one_grouped_entry():
    st = dg.gemm_strided_batched(0, 0, 8, 8, 8, 1 << 20, 8, 64, 1 << 24, 8, 64, 1 << 28, 8, 4, 3, dg.GEMM_F32,
                                 check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE and "stride_c" in dg.gemm_last_error()
    assert dg.gemm_strided_batched(0, 0, 8, 8, 8, 0, 8, 64, 0, 8, 64, 0, 8, 64, 0, dg.GEMM_F32,
                                   check=False) == dg.GEMM_OK


# ----------------------------------------------------------------------------- split K
def wplan(M, N, K, dtype="f32", ws=1 << 30, req=None, check=True, epi=None):
    return dg.gemm_plan_workspace(0, 0, M, N, K, max(1, K), max(1, N), max(1, N), dg.DTYPE_CODE[dtype], 4096, 4096,
                                  4096, 256, "gfx950", ws, req, check=check, epi=epi)


def test_split_needs_workspace():
    """Without workspace nothing splits; with it, an under-filled problem splits."""
    assert plan(256, 256, 16384, "f32")[1].split_k == 1
    # the 64 x 64 direct-copy tile in slices of whole k-tile pairs (measured 30.8 us split
    # 16 ways, against 35.9 for the register-staged 64 x 64 tile)
    st, c = wplan(256, 256, 16384)
    assert st == 0 and c.split_k > 1 and c.schedule == 8 and c.launches == 2
    assert c.workspace_bytes == c.split_k * 256 * 256 * 4
    assert c.k_chunk % (2 * c.bk) == 0 and (c.split_k - 1) * c.k_chunk < 16384 <= c.split_k * c.k_chunk
    # a machine-filling problem, or a short K, does not split (the reduction would cost more)
    assert wplan(4096, 4096, 4096, "f16")[1].split_k == 1
    assert wplan(256, 256, 256)[1].split_k == 1
    assert wplan(1024, 1024, 1024)[1].split_k == 1


def test_split_forced_and_clamped():
    st, c = wplan(200, 300, 1000, req=dg.request(split_k=3))
    assert st == 0 and c.split_k == 3
    # more slices than k-tiles: as many slices as k-tiles
    st, c = wplan(200, 300, 70, req=dg.request(split_k=8, bm=64, bn=64, variant=dg.GEMM_VARIANT_MFMA))
    assert st == 0 and c.split_k == 3 and c.k_chunk == 32
    # split_k = 1 forbids splitting even with workspace
    assert wplan(256, 256, 256, req=dg.request(split_k=1))[1].split_k == 1
    # workspace rows are padded to 4 floats
    st, c = wplan(10, 6, 4096, req=dg.request(split_k=4))
    assert st == 0 and c.workspace_bytes == 4 * 10 * 8 * 4


def test_split_errors():
    st, _ = wplan(256, 256, 256, ws=1000, req=dg.request(split_k=4), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE and "workspace" in dg.gemm_last_error()
    st, _ = wplan(256, 256, 256, req=dg.request(split_k=-1), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
    st, _ = wplan(256, 256, 256, ws=-5, check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
    # the ping-pong schedule does not split
    st, _ = wplan(4096, 4096, 4096, "f16", req=dg.request(schedule=2, split_k=2), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED
    # grouped calls do not split
    st, _ = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, [gp(64, 64, 64)], req=dg.request(split_k=2), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED
    # rejected before any device access
    ex = dg.library().gemm_ex_workspace
    assert ex(0, 0, 8, 8, 8, 1 << 20, 8, 1 << 21, 8, 1 << 22, 8, 0, None, None, -1, None) == dg.GEMM_ERR_INVALID_VALUE
    assert ex(0, 0, 8, 8, 8, 1 << 20, 8, 1 << 21, 8, 1 << 22, 8, 0, None, None, 64, None) == dg.GEMM_ERR_NULL_POINTER
    assert ex(0, 0, 0, 8, 8, 0, 8, 0, 8, 0, 8, 0, None, None, 0, None) == dg.GEMM_OK


def test_split_workspace_rejections_before_device():
    """Workspace checks cover the whole declared range and run before any device access."""
    ex = dg.library().gemm_ex_workspace
    A, B, C = 1 << 30, (1 << 30) + (1 << 22), (1 << 30) + (2 << 22)
    args = (0, 0, 256, 256, 256, A, 256, B, 256, C, 256, 0, None)
    W = (1 << 30) + (8 << 22)
    assert ex(*args, W + 4, 1 << 22, None) == dg.GEMM_ERR_INVALID_VALUE
    assert "aligned" in dg.gemm_last_error()
    for w in (A, B + 1024 * 16, C - (1 << 20)):
        assert ex(*args, w, 4 << 20, None) == dg.GEMM_ERR_INVALID_VALUE
        assert "overlaps" in dg.gemm_last_error()


# ----------------------------------------------------------------------------- packed operands
def test_pack_plan_choices():
    # the ragged bf16 benchmark problem runs directly on the register-staged
    # software-pipelined kernel; forced packing puts it on the direct-copy one, whole
    # tiles of K = 1088
    st, c = dg.gemm_plan_workspace(0, 1, 3001, 5003, 1037, 1037, 1037, 5003, dg.GEMM_BF16, 4096, 4096, 4096, 256,
                                   "gfx950", 1 << 30)
    assert st == 0 and c.pack == 1 and c.schedule == 7 and c.launches == 1
    st, c = dg.gemm_plan_workspace(0, 1, 3001, 5003, 1037, 1037, 1037, 5003, dg.GEMM_BF16, 4096, 4096, 4096, 256,
                                   "gfx950", 1 << 30, dg.request(pack=2))
    # (the packed product measured the same on the ping-pong and the software-pipelined
    # kernels: 50.4 against 50.7 us)
    assert st == 0 and c.pack == 2 and c.schedule in (2, 5) and c.vec == 1 and c.launches == 2
    assert (c.tiles_m, c.tiles_n) == (12, 20)
    assert c.workspace_bytes == 3072 * 1088 * 2 + 5120 * 1088 * 2
    # a 16-bit problem with misaligned rows and no room for the register-staged kernel's
    # 16-byte chunks (K < 8) still packs when a workspace is given
    st, c = dg.gemm_plan_workspace(0, 0, 4096, 4096, 7, 7, 4097, 4096, dg.GEMM_F16, 4096, 4096, 4096, 256,
                                   "gfx950", 1 << 30)
    assert st == 0 and c.schedule != 7
    # an aligned whole-tile problem gains nothing from a copy
    assert wplan(4096, 4096, 4096, "f16")[1].pack == 1


def test_pack_errors():
    st, _ = wplan(300, 300, 300, "f16", ws=1000, req=dg.request(pack=2), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE and "workspace" in dg.gemm_last_error()
    st, _ = wplan(300, 300, 0, "f16", req=dg.request(pack=2), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
    st, _ = wplan(300, 300, 300, "f16", req=dg.request(pack=3), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
    st, _ = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, [gp(64, 64, 64)], req=dg.request(pack=2), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED
    # 16-byte loads on a base not aligned to the element: possible only by packing
    st, _ = dg.gemm_plan(0, 0, 64, 64, 63, 63, 64, 64, dg.GEMM_F16, 1, 0, 0, req=dg.request(vec=1), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED
    st, c = dg.gemm_plan_workspace(0, 0, 64, 64, 63, 63, 64, 64, dg.GEMM_F16, 1, 0, 0, 256, "gfx950", 1 << 20,
                                   dg.request(vec=1))
    assert st == 0 and c.pack == 2 and c.vec == 1


# ----------------------------------------------------------------------------- fused epilogue
def test_epilogue_plan_avoids_plain_only_kernels():
    gelu = dg.epilogue(alpha=2.0, activation="gelu_tanh")
    st, _ = wplan(4096, 4096, 4096, "f16", req=dg.request(schedule=4), epi=gelu, check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED
    # the identity epilogue is the plain store: any kernel
    assert wplan(4096, 4096, 4096, "f16", req=dg.request(schedule=4), epi=dg.epilogue())[1].schedule == 4
    # the headline configuration keeps its software-pipelined kernel with an epilogue
    assert wplan(4096, 4096, 4096, "f16", epi=gelu)[1].schedule == 5
    st, _ = wplan(64, 64, 64, epi=dg.epilogue(out_dtype=7), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE


def test_epilogue_rejections_before_device():
    ex = dg.gemm_ex_epilogue
    A, B, C = 1 << 30, (1 << 30) + (1 << 22), (1 << 30) + (2 << 22)
    R, bias = (1 << 30) + (4 << 22), (1 << 30) + (5 << 22)
    args = (0, 0, 64, 64, 64, A, 64, B, 64, C, 64, dg.GEMM_F32)

    def call(epi, ws=None, wsb=0):
        return ex(*args, epi, None, ws, wsb, None, check=False)
    assert call(dg.epilogue(out_dtype=5)) == dg.GEMM_ERR_INVALID_VALUE
    assert call(dg.epilogue(activation=9, alpha=2.0)) == dg.GEMM_ERR_INVALID_VALUE
    assert call(dg.epilogue(beta=1.0, R=None, ldr=64)) == dg.GEMM_ERR_NULL_POINTER
    assert call(dg.epilogue(beta=1.0, R=R, ldr=10)) == dg.GEMM_ERR_INVALID_VALUE
    # R overlapping C without being C
    assert call(dg.epilogue(beta=1.0, R=C + 256, ldr=64)) == dg.GEMM_ERR_INVALID_VALUE
    assert "R overlaps C" in dg.gemm_last_error()
    # R == C with another leading dimension is not the in-place form
    assert call(dg.epilogue(beta=1.0, R=C, ldr=65)) == dg.GEMM_ERR_INVALID_VALUE
    # a leading dimension of R whose extent overflows 64 bits is refused, not wrapped
    # into a range that could slip past the overlap checks
    for ldr in ((1 << 63) - 1, 1 << 57):
        assert call(dg.epilogue(beta=1.0, R=R, ldr=ldr)) == dg.GEMM_ERR_INVALID_VALUE
        assert "extent" in dg.gemm_last_error()
    assert call(dg.epilogue(bias=C + 64, alpha=2.0)) == dg.GEMM_ERR_INVALID_VALUE
    assert "bias" in dg.gemm_last_error()
    # the workspace must not overlap the epilogue operands either
    assert call(dg.epilogue(beta=1.0, R=R, ldr=64), ws=R, wsb=1 << 16) == dg.GEMM_ERR_INVALID_VALUE
    # C in a 16-bit output type overlapping A is caught with C's own element size
    args16 = (0, 0, 64, 64, 64, A, 64, B, 64, A - 64 * 64 * 2 + 64, 64, dg.GEMM_F32)
    assert ex(*args16, dg.epilogue(out_dtype="f16", alpha=2.0), None, None, 0, None, check=False) == \
        dg.GEMM_ERR_INVALID_VALUE
    # empty output: nothing to check, nothing launched
    assert ex(0, 0, 0, 64, 64, 0, 64, 0, 64, 0, 64, 0, dg.epilogue(beta=1.0), None, None, 0, None,
              check=False) == dg.GEMM_OK


def test_threads_request_selects_k_split_kernels():
    """The fp32 64 x 64 tile exists with one wave grid (256 threads) and with two that
    split K (512 threads); the requested workgroup size picks between them."""
    for threads in (256, 512):
        st, c = plan(1024, 1024, 1024, "f32", req=dg.request(bm=64, bn=64, threads=threads))
        assert st == 0 and c.threads == threads and (c.bm, c.bn) == (64, 64)
    st, _ = plan(1024, 1024, 1024, "f32", req=dg.request(threads=-1))
    assert st == dg.GEMM_ERR_INVALID_VALUE
    st, _ = plan(1024, 1024, 1024, "f32", req=dg.request(bm=64, bn=64, threads=384))
    assert st == dg.GEMM_ERR_UNSUPPORTED
    # grouped calls have no K-split form
    st, _ = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, [dg.problem(64, 64, 64, 0x10000, 64, 0x100000, 64, 0x200000, 64)],
                                 req=dg.request(bm=64, bn=64, threads=512), check=False)
    assert st == dg.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_grouped_plan_every_variant(dtype):
    """Both kernel families have grouped forms for every input type."""
    probs = [dg.problem(100, 90, 80, 0x10000, 80, 0x100000, 90, 0x200000, 90)]
    for variant in (dg.GEMM_VARIANT_LDS, dg.GEMM_VARIANT_MFMA):
        st, c = dg.gemm_grouped_plan(0, 0, dg.DTYPE_CODE[dtype], probs, req=dg.request(variant=variant), check=False)
        assert st == 0 and c.variant == variant, (dtype, variant, dg.gemm_last_error())
