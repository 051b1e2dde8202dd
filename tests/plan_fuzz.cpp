// plan_fuzz.cpp -- randomized checks of the host-only planner (validation, the
// single-problem heuristic and the grouped heuristic). Built with the address and
// undefined-behaviour sanitizers by tests/test_plan_fuzz.py; any sanitizer report
// or broken invariant ends the run with a nonzero status.
//
// Usage: plan_fuzz SEED ITERATIONS
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <random>
#include <vector>

#include "../dense_gemm_06_amd/csrc/plan.h"

using namespace dg;

static std::mt19937_64 rng;
static int64_t pick(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }
static bool coin(int pct) { return pick(0, 99) < pct; }

// Sizes: mostly small or near multiples of the tile sizes, sometimes at or past the
// library's limits, rarely negative.
static int64_t size_value() {
    const int64_t r = pick(0, 99);
    if (r < 5) return pick(0, 3);
    if (r < 45) return pick(0, 700);
    if (r < 70) return pick(1, 40) * 256 + pick(-8, 8);
    if (r < 85) return pick(1, 1200) * 8;
    if (r < 90) return pick(1, 70000);
    if (r < 93) return pick(1, (int64_t)1 << 24);
    if (r < 97) return ((int64_t)1 << 30) + pick(-3, 3);
    return -pick(1, 5);
}

static int64_t ld_value(int64_t minimum) {
    const int64_t r = pick(0, 99);
    if (r < 35) return minimum;
    if (r < 60) return minimum + pick(0, 9);
    if (r < 85) return (minimum + 7) / 8 * 8;
    if (r < 92) return ((int64_t)1 << 23) + pick(-9, 2);
    if (r < 96) return minimum - pick(1, 3);  // too short
    return coin(50) ? ((int64_t)1 << 40) : pick(1, 100000);
}

static uintptr_t ptr_value() {
    static const int offs[] = {0, 1, 2, 3, 4, 6, 8, 12, 16, 256};
    return ((uintptr_t)pick(1, 1 << 20) << 24) + offs[pick(0, 9)];
}

static int fails = 0;
#define CHECK(cond, ...)                                                 \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "invariant failed: %s: ", #cond);            \
            fprintf(stderr, __VA_ARGS__);                                \
            fprintf(stderr, "\n");                                       \
            if (++fails > 20) exit(1);                                   \
        }                                                                \
    } while (0)

static void random_request(gemm_config* r) {
    memset(r, 0, sizeof *r);
    r->variant = (int32_t)pick(-1, 3);
    static const int tiles[] = {0, 0, 0, 32, 64, 128, 256, 96};
    r->bm = tiles[pick(0, 7)];
    r->bn = tiles[pick(0, 7)];
    r->vec = (int32_t)pick(-2, 2);
    r->xcd_remap = (int32_t)pick(-2, 2);
    r->group_m = (int32_t)(coin(70) ? 0 : pick(-1, 40));
    r->waves_m = (int32_t)(coin(70) ? 0 : pick(-1, 5));
    r->waves_n = (int32_t)(coin(70) ? 0 : pick(-1, 5));
    r->threads = (int32_t)(coin(70) ? 0 : pick(-1, 3) * 256);
    r->schedule = (int32_t)(coin(60) ? 0 : pick(-1, 10));
    r->split_k = (int32_t)(coin(60) ? 0 : pick(-1, 20));
    r->pack = (int32_t)(coin(60) ? 0 : pick(-1, 3));
    r->max_grid = (int32_t)(coin(70) ? 0 : pick(-1, 600));
    r->stream_k = (int32_t)(coin(60) ? 0 : pick(-1, 3));
    r->sk_width = (int32_t)(coin(70) ? 0 : pick(-1, 600));
}

static void check_plan(int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int dtype, uintptr_t a,
                       uintptr_t b, int64_t ws, bool epi, const gemm_config* req, const gemm_config& c, int cus) {
    CHECK(c.kernel_id >= 0 && c.kernel_id < kMenuSize, "kernel %d", c.kernel_id);
    if (c.kernel_id < 0 || c.kernel_id >= kMenuSize) return;
    const MenuEntry& e = kMenu[c.kernel_id];
    const int es = dtype == 0 ? 4 : 2;
    const bool packed = c.pack == 2;
    CHECK(e.dtype == dtype && e.opb == opB, "entry %d dtype %d opb %d for %d %d", e.id, e.dtype, e.opb, dtype, opB);
    CHECK(c.bm == e.bm && c.bn == e.bn && c.bk == e.bk && c.schedule == e.sched && c.threads == e.threads,
          "config does not match entry %d", e.id);
    CHECK(schedule_enabled(e.sched), "switched-off schedule %d chosen", e.sched);
    CHECK(!epi || epilogue_capable(e.sched), "schedule %d with an epilogue", e.sched);
    CHECK(c.split_k >= 1 && (c.split_k == 1 || e.sched == 1 || e.sched == 5 || e.sched == 7 || e.sched == 8 || e.sched == 9), "split %d on schedule %d", c.split_k, e.sched);
    CHECK(c.split_k == 1 || e.sched != 8 || c.k_chunk % 64 == 0, "schedule 8 slice of %lld", (long long)c.k_chunk);
    CHECK(c.split_k == 1 || c.grid == c.tiles_m * c.tiles_n, "split %d on a persistent grid", c.split_k);
    CHECK(!(c.split_k > 1 && packed), "split and packed");
    CHECK(c.workspace_bytes >= 0 && c.workspace_bytes <= (ws > 0 ? ws : 0), "workspace %lld of %lld",
          (long long)c.workspace_bytes, (long long)ws);
    const bool sk = c.stream_k == 2;
    CHECK(c.stream_k == 1 || c.stream_k == 2, "stream_k out %d", c.stream_k);
    CHECK(c.launches == ((c.split_k > 1 || packed || sk) ? 2 : 1), "launches %d", c.launches);
    CHECK(!req || req->stream_k != 1 || !sk, "stream-K used with stream_k = 1");
    CHECK(!req || req->stream_k != 2 || sk, "stream_k = 2 accepted without stream-K");
    if (sk) {
        // the 8-wave persistent software-pipelined kernel on whole k-tiles, at least 8 of
        // them; no packing or split; sk_width above the tail's tiles and at most the
        // grid, shares of at least 4 k-tiles, 512 KiB of workspace per sharing workgroup
        const int64_t tiles = c.tiles_m * c.tiles_n;
        const int64_t S = tiles > c.grid ? tiles % c.grid : tiles;
        const int64_t KT = K / 32;
        CHECK(e.sched == 5 && e.threads == 512 && !packed && c.split_k == 1 && K % 32 == 0 && KT >= 8,
              "stream-K on schedule %d, K %lld", e.sched, (long long)K);
        CHECK(S > 0 && S < c.grid && c.sk_width > S && c.sk_width <= c.grid && (S * KT) / c.sk_width >= kSkMinPiece,
              "stream-K tail %lld on %d of grid %d, KT %lld", (long long)S, c.sk_width, c.grid, (long long)KT);
        CHECK(c.workspace_bytes == (int64_t)c.sk_width * 524288, "stream-K workspace %lld", (long long)c.workspace_bytes);
        CHECK(!req || req->max_grid <= 0 || c.grid == req->max_grid, "stream-K grid %d, max_grid %d", c.grid,
              req ? req->max_grid : 0);
        CHECK(!req || req->sk_width <= 0 || c.sk_width == req->sk_width, "sk_width %d asked %d", c.sk_width,
              req ? req->sk_width : 0);
    } else {
        CHECK(c.sk_width == 0, "sk_width %d without stream-K", c.sk_width);
    }
    CHECK(std::isfinite(c.est_cycles) && c.est_cycles >= 0, "estimate %g", c.est_cycles);
    if (M > 0 && N > 0) {
        CHECK(c.tiles_m >= 1 && c.tiles_n >= 1 && c.tiles_m * c.bm >= M && c.tiles_n * c.bn >= N,
              "tiles %lld x %lld of %d x %d for %lld x %lld", (long long)c.tiles_m, (long long)c.tiles_n, c.bm, c.bn,
              (long long)M, (long long)N);
        // one workgroup per tile, or a persistent grid of the 8-wave software-pipelined
        // kernel on whole k-tiles (padded K when packed), no split: the requested cap,
        // or without one a workgroup per compute unit (one fits per unit)
        const int64_t tiles = c.tiles_m * c.tiles_n;
        const int64_t Kx = packed ? (K + 63) / 64 * 64 : K;
        const bool capped = req && req->max_grid > 0;
        CHECK((int64_t)c.grid == tiles ||
                  ((c.grid < tiles || sk) && persistent_capable(e.sched, e.threads, Kx) && c.split_k == 1 &&
                   c.grid == (capped ? req->max_grid : cus)),
              "grid %d for %lld tiles (max_grid %d, schedule %d, K %lld)", c.grid, (long long)tiles,
              req ? req->max_grid : 0, e.sched, (long long)K);
        if (req && req->max_grid > 0) CHECK(c.grid <= req->max_grid, "grid %d above max_grid %d", c.grid, req->max_grid);
    }
    if (e.vec && !packed) CHECK(a % es == 0 && b % es == 0, "16-byte loads on bases not aligned to the element");
    if (direct_copy(e.sched) && !packed) {
        CHECK(a % 16 == 0 && b % 16 == 0 && (lda * es) % 16 == 0 && (ldb * es) % 16 == 0,
              "direct copies on unaligned operands");
        CHECK(K > 0 && K % 8 == 0, "direct copies with K = %lld", (long long)K);
        if (e.sched != 5) CHECK(K % e.bk == 0, "schedule %d with K = %lld", e.sched, (long long)K);
        if (e.sched == 8) CHECK(K % 64 == 0, "schedule 8 with K = %lld", (long long)K);
        if (opB == 0)
            CHECK(N % e.bn == 0 || N % (e.sched == 8 || e.sched == 9 ? 4 : 8) == 0, "row-major B edge tile with N = %lld",
                  (long long)N);
    }
    if (e.sched == 7) {
        // whole 16-byte chunks inside every row: K >= 8, N >= 8 for a row-major B, and
        // 16-byte loads (element-aligned bases unless packed)
        CHECK(e.vec == 1 && K >= 8 && (opB == 1 || N >= 8 || (packed && N > 0)),
              "register-staged software-pipelined kernel with K = %lld, N = %lld", (long long)K, (long long)N);
    }
    if (req) {
        if (req->bm) CHECK(c.bm == req->bm, "bm %d requested %d", c.bm, req->bm);
        if (req->bn) CHECK(c.bn == req->bn, "bn %d requested %d", c.bn, req->bn);
        if (req->schedule) CHECK(c.schedule == req->schedule, "schedule %d requested %d", c.schedule, req->schedule);
        if (req->threads) CHECK(c.threads == req->threads, "threads");
        if (req->variant) CHECK(c.variant == req->variant, "variant");
        if (req->vec >= 0) CHECK(c.vec == req->vec, "vec");
        if (req->split_k >= 2) CHECK(c.split_k >= 1 && c.split_k <= req->split_k, "split %d requested %d",
                                     c.split_k, req->split_k);
        if (req->pack == 1) CHECK(!packed, "packed against pack = 1");
        if (req->pack == 2) CHECK(packed, "not packed against pack = 2");
    }
}

int main(int argc, char** argv) {
    const uint64_t seed = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
    const long iters = argc > 2 ? strtol(argv[2], nullptr, 10) : 20000;
    rng.seed(seed);
    long ok = 0, rejected = 0;
    for (long it = 0; it < iters; ++it) {
        const int opA = coin(95) ? 0 : (int)pick(-1, 2);
        const int opB = coin(95) ? (int)pick(0, 1) : (int)pick(-1, 2);
        const int dtype = coin(95) ? (int)pick(0, 2) : (int)pick(-1, 4);
        const int64_t M = size_value(), N = size_value(), K = size_value();
        const int64_t lda = ld_value(K > 0 ? K : 1);
        const int64_t ldb = ld_value(opB == 1 ? (K > 0 ? K : 1) : (N > 0 ? N : 1));
        const int64_t ldc = ld_value(N > 0 ? N : 1);
        const uintptr_t a = ptr_value(), b = ptr_value(), cp = ptr_value();
        const int cus = coin(90) ? 256 : (int)pick(-1, 400);
        const char* arch = coin(95) ? "gfx950" : (coin(50) ? "gfx942" : nullptr);
        const int64_t ws = coin(50) ? 0 : (coin(80) ? pick(0, (int64_t)1 << 34) : pick(-5, 5));
        const bool epi = coin(20);
        gemm_config req, out;
        const bool with_req = coin(50);
        if (with_req) random_request(&req);
        memset(&out, 0x5a, sizeof out);
        const int st = plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a, b, cp, cus, arch, ws, epi,
                            with_req ? &req : nullptr, &out);
        CHECK(st >= GEMM_OK && st <= GEMM_ERR_LAUNCH, "status %d", st);
        if (st == GEMM_OK) {
            ++ok;
            check_plan(opB, M, N, K, lda, ldb, dtype, a, b, ws, epi, with_req ? &req : nullptr, out, cus);
            // the same call again (now answered by the plan cache, or after another
            // entry took its slot) gives the same plan
            gemm_config again;
            memset(&again, 0x33, sizeof again);
            const int st2 = plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a, b, cp, cus, arch, ws, epi,
                                 with_req ? &req : nullptr, &again);
            CHECK(st2 == GEMM_OK && memcmp(&again, &out, sizeof out) == 0, "repeated plan differs (status %d)", st2);
        } else {
            ++rejected;
            CHECK(last_error() && last_error()[0], "status %d without a message", st);
        }

        // grouped: a few problems around the same sizes
        if (it % 4 == 0) {
            const int count = (int)pick(-1, 6);
            std::vector<gemm_problem> probs((size_t)(count > 0 ? count : 1));
            for (int i = 0; i < count; ++i) {
                gemm_problem& p = probs[(size_t)i];
                p.M = coin(70) ? pick(0, 600) : size_value();
                p.N = coin(70) ? pick(0, 600) : size_value();
                p.K = coin(70) ? pick(0, 600) : size_value();
                p.lda = ld_value(p.K > 0 ? p.K : 1);
                p.ldb = ld_value(opB == 1 ? (p.K > 0 ? p.K : 1) : (p.N > 0 ? p.N : 1));
                p.ldc = ld_value(p.N > 0 ? p.N : 1);
                p.A = (const void*)ptr_value();
                p.B = (const void*)ptr_value();
                p.C = (float*)ptr_value();
                p.batch = coin(70) ? 1 : pick(-1, 5);
                p.stride_a = pick(-1, 1 << 22);
                p.stride_b = pick(-1, 1 << 22);
                p.stride_c = pick(-1, 1 << 22);
            }
            gemm_config g;
            memset(&g, 0x5a, sizeof g);
            const int gst = plan_grouped(opA, opB, dtype, count > 0 ? probs.data() : nullptr, count, cus, arch,
                                         with_req ? &req : nullptr, &g);
            CHECK(gst >= GEMM_OK && gst <= GEMM_ERR_LAUNCH, "grouped status %d", gst);
            if (gst == GEMM_OK && g.kernel_id >= 0) {
                CHECK(g.kernel_id < kMenuSize, "grouped kernel %d", g.kernel_id);
                if (g.kernel_id < kMenuSize) {
                    const MenuEntry& e = kMenu[g.kernel_id];
                    CHECK(grouped_capable(e.variant, e.sched, e.bm, e.bn, e.wm, e.wn, e.threads),
                          "grouped run of entry %d", e.id);
                    CHECK(e.dtype == dtype && e.opb == opB, "grouped entry dtype/opb");
                    CHECK((g.grid >= 1) == (g.tiles_total > 0) && (g.launches == (g.tiles_total > 0 ? 1 : 0)),
                          "grouped grid %d for %lld tiles, %d launches", g.grid, (long long)g.tiles_total, g.launches);
                    CHECK(!with_req || req.max_grid <= 0 || g.grid <= req.max_grid,
                          "grouped grid %d above max_grid %d", g.grid, req.max_grid);
                }
            } else if (gst != GEMM_OK) {
                CHECK(last_error() && last_error()[0], "grouped status %d without a message", gst);
            }
        }
    }
    printf("ok %ld plans accepted, %ld rejected, %d invariant failures\n", ok, rejected, fails);
    return fails ? 1 : 0;
}
