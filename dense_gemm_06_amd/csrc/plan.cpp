// plan.cpp -- argument validation and the launch heuristic (host only, no HIP).
//
// The heuristic plays the role of gpu_opt_choice in "GPU architecture and
// mapping kernels" (section 12.9) for one operation, C = A @ B: threads are laid
// out along the contiguous axis (fixed inside each kernel), tiles are powers of
// two with masked edges instead of a divisibility requirement, a register
// micro-tile (or MFMA wave tile) is always used because the kernel reduces, and
// the grid must fill the machine (the chapter's exercise on a minimum block
// count): among the compiled configurations it picks the one with the lowest
// estimated time, where the estimate counts how many rounds of workgroups the
// 256 compute units need. 16-byte global loads are used only when the operand
// bases and leading dimensions are 16-byte aligned (the learn-cutedsl README's
// point that vector copies need a known 16-byte alignment).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include <algorithm>
#include <cmath>
#include <string>

#include "../../include/gemm.h"
#include "menu.h"
#include "plan.h"

namespace dg {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
}
void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }

const MenuEntry kMenu[kMenuSize] = {
#define DG_ENTRY(id, variant, dtype, opb, vec, bm, bn, bk, wm, wn, tm, tn, threads, lds, sched) \
    {id, variant, dtype, opb, vec, bm, bn, bk, wm, wn, tm, tn, threads, lds, sched},
    DG_MENU(DG_ENTRY)
#undef DG_ENTRY
};

bool extent_fits(int64_t rows, int64_t cols, int64_t ld) {
    if (rows <= 0 || cols <= 0) return true;
    const unsigned __int128 n = (unsigned __int128)(uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols;
    return (n * 4) >> 62 == 0;
}

static const char* dtype_name(int dt) { return dt == 0 ? "fp32" : dt == 1 ? "fp16" : "bf16"; }
static int elem_size(int dt) { return dt == DT_F32 ? 4 : 2; }

int validate(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
             int dtype) {
    if (dtype < 0 || dtype > 2) {
        set_error("dtype %d is not GEMM_F32 (0), GEMM_F16 (1) or GEMM_BF16 (2)", dtype);
        return GEMM_ERR_INVALID_VALUE;
    }
    if ((opA != GEMM_OP_N && opA != GEMM_OP_T) || (opB != GEMM_OP_N && opB != GEMM_OP_T)) {
        set_error("opA = %d / opB = %d: operand flags must be GEMM_OP_N (0) or GEMM_OP_T (1)", opA, opB);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (M < 0 || N < 0 || K < 0) {
        set_error("negative size: M = %lld, N = %lld, K = %lld", (long long)M, (long long)N, (long long)K);
        return GEMM_ERR_INVALID_VALUE;
    }
    const int64_t minlda = std::max<int64_t>(1, K);
    const int64_t minldb = opB == GEMM_OP_N ? std::max<int64_t>(1, N) : std::max<int64_t>(1, K);
    const int64_t minldc = std::max<int64_t>(1, N);
    if (lda < minlda) {
        set_error("lda = %lld is smaller than max(1, K) = %lld", (long long)lda, (long long)minlda);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (ldb < minldb) {
        set_error("ldb = %lld is smaller than %s = %lld", (long long)ldb,
                  opB == GEMM_OP_N ? "max(1, N) for row-major B" : "max(1, K) for column-major B",
                  (long long)minldb);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (ldc < minldc) {
        set_error("ldc = %lld is smaller than max(1, N) = %lld", (long long)ldc, (long long)minldc);
        return GEMM_ERR_INVALID_VALUE;
    }
    // C's element range, (M - 1) * ldc + N elements of up to 4 bytes, must be
    // representable (the overlap checks and the kernels' 64-bit offsets rely on it)
    if (!extent_fits(M, N, ldc)) {
        set_error("ldc = %lld: C's extent (M - 1) * ldc + N (M = %lld, N = %lld) does not fit in the address space",
                  (long long)ldc, (long long)M, (long long)N);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (opA == GEMM_OP_T) {
        set_error("opA = GEMM_OP_T (column-major A) is not implemented by this library");
        return GEMM_ERR_UNSUPPORTED;
    }
    // The kernels index rows, columns and k with 32-bit integers (tile origins
    // plus one tile of slack must stay representable).
    const int64_t lim = (int64_t)1 << 30;
    if (M >= lim || N >= lim || K >= lim) {
        set_error("sizes must be below 2^30 (M = %lld, N = %lld, K = %lld)", (long long)M, (long long)N,
                  (long long)K);
        return GEMM_ERR_UNSUPPORTED;
    }
    // Per-thread global offsets are 32-bit: up to 256 rows of a leading dimension.
    const int64_t ldlim = (int64_t)1 << 23;
    if (lda >= ldlim || ldb >= ldlim) {
        set_error("leading dimensions must be below 2^23 elements (lda = %lld, ldb = %lld)", (long long)lda,
                  (long long)ldb);
        return GEMM_ERR_UNSUPPORTED;
    }
    if ((M + 255) / 256 * ((N + 255) / 256) >= lim || ((M + 63) / 64) * ((N + 63) / 64) >= ((int64_t)1 << 31)) {
        set_error("too many output tiles for one launch (M = %lld, N = %lld)", (long long)M, (long long)N);
        return GEMM_ERR_UNSUPPORTED;
    }
    return GEMM_OK;
}

// Matrix throughput per compute unit per clock and a per-tile efficiency
// factor (smaller tiles reuse each loaded byte fewer times and leave the
// matrix units waiting on LDS and global memory more often).
static double rate_per_cu(const MenuEntry& e) {
    if (e.variant == V_LDS) return 128.0;  // 64 lanes x 2 FLOP per FMA, one wave64 FMA per SIMD per 4 clocks x 4 SIMDs
    return e.dtype == DT_F32 ? 256.0 : 4096.0;
}
static double tile_efficiency_aligned(const MenuEntry& e);
// Per-tile efficiency of the kernels without a fitted time (the SIMT kernels, the
// grouped kernels and 16-bit element-wise loads) and a load-path factor: 16-byte
// loads from rows that are not 16-byte aligned, on the register-staged 256 x 256
// kernels, as measured against the same kernel on a 16-byte-aligned problem of the
// same tile counts: 16-bit 3001 x 5003 x 1037 with column-major B 69-75 us against
// 54-57 (3008 x 5008 x 1040), 4095^3 f16 310-321 us against 165 (4096^3).
// Element-wise loads (bases not aligned to the element) measured about 3x slower
// for 16-bit inputs and are assumed 1.7x slower for fp32.
static double tile_efficiency(const MenuEntry& e, bool rows16) {
    const bool f32 = e.dtype == DT_F32;
    const double load = !e.vec ? (f32 ? 0.6 : 0.35) : (rows16 || e.sched == 7) ? 1.0 : (f32 ? 0.8 : 0.55);
    return tile_efficiency_aligned(e) * load;
}
static double tile_efficiency_aligned(const MenuEntry& e) {
    const int t = std::min(e.bm, e.bn);
    // measured at 4096^3 fp16: ping-pong 144 us, software-pipelined 164 us,
    // register-staged 256 x 256 165 us
    if (e.sched == 2) return 0.97;
    if (e.sched == 4) return 0.96;
    if (e.sched == 5 || e.sched == 7) return 0.90;  // problem-dependent: see plan()
    if (e.variant == V_LDS) return t >= 128 ? 0.6 : 0.35;
    return t >= 256 ? 0.85 : t >= 128 ? 0.7 : 0.45;
}
// Time model of the MFMA tile families (fitted, in us, per family): the larger of a
// per-CU bound, rounds of tiles of `resident` tiles each at a per-CU rate (16-bit:
// min(resident r1, rcap) TFLOP/s; fp32: a rate per resident count) plus a fixed a
// per round, and a chip bound c + 2MNK / R (for 16-bit inputs the board's power
// limit: a problem that keeps every CU busy runs at R TFLOP/s whatever its tile). The
// per-CU bound is what makes few tiles of long K slow, and R what makes the largest
// tiles win once the machine is full. ks stretches the k loop for rows that are not
// 16-byte aligned (fp32; the 16-bit register-staged kernels take a fixed factor, see
// plan()).
//
// 16-bit families on 16-byte loads: 1290 medians of five alternated passes over 26
// shapes of 512 to 8192 and 120 more between 512^2 x 256 and 8192^2 x 16384, both B
// layouts, one box, splits included; median error 1.6-6.8% per family.
//
// fp32 families, per B layout: 1694 medians of five passes in shuffled order over 28
// shapes of 256^2 x 4096 to 8192^2 x 512, both B layouts, every tile with and without
// K split 2-16 ways, and 8 shapes with A rows one element off 16-byte alignment, and
// 180 medians of seven passes on 90 shapes drawn at random (log-uniform 256-8192, a
// third of them ragged); median error 0.3-3.3% per family and layout (the per-tile
// efficiency model used before: 3-47%). A partial tile in M or N stretches the
// register-staged tiles' k loop by 4-33% (edge): an edge tile's masked loads run at
// up to half speed and, a round of tiles ending together, set the launch's time
// (1024 x 1028 x 4096 on 64 x 64 tiles 228 us, against 160 for 1024 x 1088). The 64 x 64 four-wave tile runs its k loop at 0.35, 0.43, 0.46 and
// 0.47 TFLOP/s per CU with one to four resident (a shared cap reached at two
// resident had it 35% off at 1280^2 x 8192), and the chip bound takes over at five;
// the direct-copy 256 x 128 tile's k loop is the faster with row-major B (0.562
// against 0.543), the 128 x 128 tile's with column-major B (0.560 against 0.545);
// rows that are not 16-byte aligned cost the register-staged fp32 tiles 2-5% (not
// the 25% assumed before).
struct TimeFit {
    double a, r1, rcap, c, R, ks;
    double edge;     // k-loop stretch when M or N leaves a partial tile (register-staged fp32 tiles)
    double rate[5];  // if set: the per-CU rate with 1, 2, ... resident tiles (fp32)
};
static const TimeFit* time_fit(const MenuEntry& e) {
    static const TimeFit rs64{3.25, 1.12, 2.90, 4.52, 537.4, 1, 1}, rs128{5.97, 2.77, 4.00, 4.46, 834.0, 1, 1},
        rs256{14.79, 5.18, 5.18, 6.12, 900.4, 1, 1}, wide{15.34, 4.16, 4.16, 7.10, 802.7, 1, 1},
        pp16{14.61, 6.84, 6.84, 6.34, 1065.8, 1, 1}, pp32{16.96, 6.39, 6.39, 5.09, 927.8, 1, 1},
        sp4{17.35, 8.72, 8.72, 11.69, 1086.0, 1, 1}, sp8{13.36, 9.23, 9.23, 8.18, 1108.1, 1, 1},
        spr8{14.69, 7.65, 7.65, 11.31, 1011.2, 1, 1};
    // fp32, per B layout (row-major, column-major): register-staged 64 x 64 on four
    // waves (five resident per CU) and on two K groups (two), 128 x 128 (two), 256 x 128
    // (one), 16 x 64 with four K groups (two); the three-stage 256 x 128 and 64 x 64
    // tiles; the direct-copy 64 x 64, 256 x 128 and 128 x 128 tiles (one resident
    // each). The unaligned runs had row-major B; both layouts take their ks.
    static const TimeFit f_rs64[2]{{2.75, 0, 0, 6.37, 120.7, 1.031, 1.223, {0.3497, 0.4330, 0.4562, 0.4656, 0.6140}}, {2.41, 0, 0, 5.53, 119.3, 1.031, 1.165, {0.3615, 0.4437, 0.4748, 0.4678, 0.6140}}},
        f_kg2[2]{{2.56, 0, 0, 6.74, 117.1, 1.034, 1.213, {0.3985, 0.5001}}, {2.11, 0, 0, 5.72, 115.0, 1.034, 1.163, {0.3868, 0.4823}}},
        f_rs128[2]{{7.52, 0, 0, 10.71, 129.0, 1.021, 1.335, {0.4865, 0.5930}}, {5.30, 0, 0, 7.15, 130.0, 1.021, 1.191, {0.4893, 0.5780}}},
        f_rs256[2]{{13.07, 0, 0, 32.25, 138.1, 1.041, 1.186, {0.5553}}, {7.40, 0, 0, 15.55, 133.2, 1.041, 1.070, {0.5338}}},
        f_s3[2]{{13.94, 0, 0, 33.74, 138.3, 1.028, 1.200, {0.5577}}, {8.46, 0, 0, 18.29, 136.7, 1.028, 1.065, {0.5427}}},
        f_s3_64[2]{{4.57, 0, 0, 4.77, 106.0, 1.021, 1.089, {0.4365}}, {2.47, 0, 0, 10.07, 150.5, 1.021, 1.035, {0.4175}}},
        f_small[2]{{2.14, 0, 0, 5.86, 83.0, 1.051, 1.614, {0.2144, 0.3372}}, {2.18, 0, 0, 5.51, 80.6, 1.051, 1.000, {0.2141, 0.3261}}},
        f_d[2]{{3.45, 0, 0, 5.45, 125.7, 1.000, 1.000, {0.4998}}, {2.85, 0, 0, 4.74, 124.0, 1.000, 1.000, {0.5010}}},
        f_w[2]{{12.69, 0, 0, 14.07, 135.0, 1.000, 1.000, {0.5621}}, {8.15, 0, 0, 8.17, 134.2, 1.000, 1.000, {0.5430}}},
        f_n[2]{{7.25, 0, 0, 10.92, 133.9, 1.000, 1.000, {0.5444}}, {5.58, 0, 0, 8.52, 139.6, 1.000, 1.000, {0.5588}}};
    if (e.variant != V_MFMA) return nullptr;
    if (e.dtype == DT_F32) {
        const int b = e.opb;
        switch (e.sched) {
            case 1:
                if (e.bm == 64 && e.bn == 64) return e.threads == 256 ? &f_rs64[b] : &f_kg2[b];
                if (e.bm == 128 && e.bn == 128) return &f_rs128[b];
                if (e.bm == 256 && e.bn == 128) return &f_rs256[b];
                if (e.bm == 16 && e.bn == 64) return &f_small[b];
                return nullptr;
            case 6: return e.bm == 256 ? &f_s3[b] : &f_s3_64[b];
            case 8: return &f_d[b];
            case 9: return e.bm == 256 ? &f_w[b] : &f_n[b];
            default: return nullptr;
        }
    }
    if (!e.vec) return nullptr;
    switch (e.sched) {
        case 1:
            if (e.bm == 64 && e.bn == 64 && e.threads == 256) return &rs64;
            if (e.bm == 128 && e.bn == 128 && e.threads == 256) return &rs128;
            if (e.bm == 256 && e.bn == 256) return e.threads == 512 ? &rs256 : &wide;
            return nullptr;
        case 2: return &pp16;
        case 4: return &pp32;
        case 5: return e.threads == 512 ? &sp8 : &sp4;
        case 7: return e.threads == 512 ? &spr8 : &sp4;  // the 4-wave form: sp4, 10% slower
        default: return nullptr;
    }
}
// kslow stretches the k loop only (slower loads), not the fixed costs.
static double fit_us(const TimeFit& f, const MenuEntry& e, int64_t rounds, int64_t resident, int64_t kt,
                     double flops, double kslow) {
    const double w = 2.0 * e.bm * e.bn * e.bk / 1e6;  // MFLOP per k-tile of one tile
    const double rate = f.rate[0] > 0 ? f.rate[std::min<int64_t>(resident, 5) - 1] : std::min((double)resident * f.r1, f.rcap);
    const double per_cu = (double)rounds * (f.a + kslow * (double)kt * (double)resident * w / rate);
    return std::max(per_cu, f.c + kslow * flops / (f.R * 1e6));
}
// Model cycles per us: the 16-bit model's (the software-pipelined 4096^3 kernel's cost
// against its time) and the fp32 model's, to set fitted times beside the families the
// fits do not cover (the SIMT kernels).
constexpr double kCycles16PerUs = 1141.0;
constexpr double kCycles32PerUs = 2900.0;

static int blocks_per_cu(const MenuEntry& e) {
    const int by_lds = (160 * 1024) / e.lds_bytes;
    const int by_waves = 32 / (e.threads / 64);  // 8 waves per SIMD x 4 SIMDs
    return std::max(1, std::min(by_lds, by_waves));
}

static bool aligned16(uintptr_t a) { return (a & 15) == 0; }
static bool elem_aligned(uintptr_t a, int es) { return (a & (uintptr_t)(es - 1)) == 0; }

void pack_dims(int64_t M, int64_t N, int64_t K, int64_t* Mp, int64_t* Np, int64_t* Kp) {
    *Mp = (M + 255) / 256 * 256;
    *Np = (N + 255) / 256 * 256;
    *Kp = (K + 63) / 64 * 64;
}

int64_t pack_a_bytes(int dtype, int64_t M, int64_t N, int64_t K) {
    int64_t Mp, Np, Kp;
    pack_dims(M, N, K, &Mp, &Np, &Kp);
    return (Mp * Kp * elem_size(dtype) + 255) / 256 * 256;
}

int64_t pack_workspace(int opB, int dtype, int64_t M, int64_t N, int64_t K) {
    (void)opB;  // K x Np (row-major B) and Np x K (column-major B) hold the same count
    int64_t Mp, Np, Kp;
    pack_dims(M, N, K, &Mp, &Np, &Kp);
    return pack_a_bytes(dtype, M, N, K) + Np * Kp * elem_size(dtype);
}

// Workspace of an S-slice split: one fp32 plane of M x round_up(N, 4) per slice.
static int64_t split_workspace(int64_t S, int64_t M, int64_t N) { return S * M * ((N + 3) / 4 * 4) * 4; }

static int plan_uncached(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                         int dtype, uintptr_t a, uintptr_t b, int num_cus, const char* arch, int64_t ws_bytes,
                         bool fused_epilogue, const gemm_config* req, gemm_config* out) {
    int st = validate(opA, opB, M, N, K, lda, ldb, ldc, dtype);
    if (st != GEMM_OK) return st;
    if (arch == nullptr || strncmp(arch, "gfx950", 6) != 0) {
        set_error("device architecture '%s' is not gfx950; the kernels are built for gfx950 only",
                  arch ? arch : "(null)");
        return GEMM_ERR_DEVICE;
    }
    if (num_cus <= 0) {
        set_error("compute-unit count %d must be positive", num_cus);
        return GEMM_ERR_INVALID_VALUE;
    }
    const int es = elem_size(dtype);
    // Register-staged kernels read 16-byte chunks with under-aligned vector loads,
    // which need only element-aligned bases; the direct global -> LDS copies of the
    // whole-tile kernels need 16-byte-aligned bases and rows.
    const bool vec_ok = elem_aligned(a, es) && elem_aligned(b, es);
    const bool dma_ok = aligned16(a) && aligned16(b) && (lda * es) % 16 == 0 && (ldb * es) % 16 == 0;

    int want_variant = GEMM_VARIANT_AUTO, want_bm = 0, want_bn = 0, want_vec = -1, want_remap = -1, want_group = 0;
    int want_wm = 0, want_wn = 0, want_sched = 0, want_split = 0, want_pack = 0, want_threads = 0, want_grid = 0;
    int want_sk = 0, want_skw = 0;
    if (ws_bytes < 0) {
        set_error("workspace_bytes = %lld must be non-negative", (long long)ws_bytes);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (req) {
        want_split = req->split_k;
        if (want_split < 0) {
            set_error("split_k = %d must be non-negative", want_split);
            return GEMM_ERR_INVALID_VALUE;
        }
        want_variant = req->variant;
        want_bm = req->bm;
        want_bn = req->bn;
        want_vec = req->vec;
        want_remap = req->xcd_remap;
        want_group = req->group_m;
        want_wm = req->waves_m;
        want_wn = req->waves_n;
        want_sched = req->schedule;
        want_threads = req->threads;
        if (want_threads < 0) {
            set_error("threads = %d must be non-negative", want_threads);
            return GEMM_ERR_INVALID_VALUE;
        }
        want_grid = req->max_grid;
        if (want_grid < 0) {
            set_error("max_grid = %d must be non-negative", want_grid);
            return GEMM_ERR_INVALID_VALUE;
        }
        if (want_sched < 0 || want_sched > 9 || want_wm < 0 || want_wn < 0 || want_variant < 0 || want_variant > 2 || want_vec < -1 || want_vec > 1 || want_remap < -1 ||
            want_remap > 1 || want_group < 0 || want_bm < 0 || want_bn < 0) {
            set_error("invalid requested configuration (variant %d, bm %d, bn %d, vec %d, xcd_remap %d, group_m %d)",
                      want_variant, want_bm, want_bn, want_vec, want_remap, want_group);
            return GEMM_ERR_INVALID_VALUE;
        }
        if (want_sched && !schedule_enabled(want_sched)) {
            set_error("schedule %d is not available: its kernel was removed from this library", want_sched);
            return GEMM_ERR_UNSUPPORTED;
        }
        want_pack = req->pack;
        if (want_pack < 0 || want_pack > 2) {
            set_error("pack = %d must be 0 (heuristic), 1 (never) or 2 (always)", want_pack);
            return GEMM_ERR_INVALID_VALUE;
        }
        want_sk = req->stream_k;
        want_skw = req->sk_width;
        if (want_sk < 0 || want_sk > 2 || want_skw < 0) {
            set_error("stream_k = %d must be 0 (heuristic), 1 (never) or 2 (always), sk_width = %d non-negative",
                      want_sk, want_skw);
            return GEMM_ERR_INVALID_VALUE;
        }
        if (want_vec == 1 && !vec_ok && (ws_bytes == 0 || want_pack == 1)) {
            set_error("16-byte loads requested but the A/B bases are not aligned to the element size");
            return GEMM_ERR_UNSUPPORTED;
        }
    }

    // Packed operands: zero-padded, aligned copies in the workspace (whole 256 x 256
    // tiles, K a multiple of 64), made by one extra launch whose traffic is charged.
    int64_t Mp, Np, Kp;
    pack_dims(M, N, K, &Mp, &Np, &Kp);
    const int64_t pack_need = pack_workspace(opB, dtype, M, N, K);
    const bool pack_fits = K > 0 && pack_need <= ws_bytes && Kp < ((int64_t)1 << 23) && Np < ((int64_t)1 << 23);
    if (want_pack == 2 && !pack_fits) {
        set_error("pack = 2 needs K > 0 and %lld bytes of workspace; %lld were given", (long long)pack_need,
                  (long long)ws_bytes);
        return GEMM_ERR_INVALID_VALUE;
    }
    const double pack_cycles =
        (double)((M * K + K * N) + (Mp * Kp + Np * Kp)) * es / 2048.0 + 16000.0;

    const MenuEntry* best = nullptr;
    double best_cost = 0;
    int64_t best_split = 1, best_chunk = K, short_ws = -1, best_grid = 0, best_sk = 0, best_skw = 0;
    bool best_packed = false;
    for (int pass = 0; pass < 2; ++pass) {
    const bool packed = pass == 1;
    if (packed ? (!pack_fits || want_pack == 1 || want_split >= 2) : want_pack == 2) continue;
    const int64_t Mx = packed ? Mp : M, Nx = packed ? Np : N, Kx = packed ? Kp : K;
    for (const MenuEntry& e : kMenu) {
        if (e.dtype != dtype || e.opb != opB) continue;
        if (want_variant != GEMM_VARIANT_AUTO && e.variant != want_variant) continue;
        if (want_bm && e.bm != want_bm) continue;
        if (want_bn && e.bn != want_bn) continue;
        if (want_wm && (e.variant == V_MFMA ? e.wm : 1) != want_wm) continue;
        if (want_sched && e.sched != want_sched) continue;
        if (want_threads && e.threads != want_threads) continue;
        if (!schedule_enabled(e.sched)) continue;
        if (fused_epilogue && !epilogue_capable(e.sched)) continue;
        // the direct-copy kernels copy whole tiles: no masking of M, N or K edges on
        // the operands (the packed copies are whole tiles; C is masked at the store).
        // The software-pipelined and ping-pong kernels also take edge tiles in M and N,
        // copying clamped rows and columns (row-major B: N a multiple of 8, so that no
        // 16-byte chunk reaches past the end of a row); the software-pipelined kernel
        // also a partial last k-tile (K a multiple of 8, zeroed past K in LDS).
        if (direct_copy(e.sched) && (Kx == 0 || (Kx % e.bk != 0 && !(e.sched == 5 && Kx % 8 == 0)))) continue;
        if (direct_copy(e.sched) && (Mx % e.bm != 0 || Nx % e.bn != 0) &&
            !((e.sched == 5 || e.sched == 2 || e.sched == 4) && (e.opb == 1 || Nx % 8 == 0)) &&
            !((e.sched == 8 || e.sched == 9) && (e.opb == 1 || Nx % 4 == 0)))
            continue;
        // the fp32 direct-copy tile: K in whole k-tiles for each of its two K groups
        if (e.sched == 8 && Kx % 64 != 0) continue;
        // the register-staged software-pipelined kernel reads whole 16-byte chunks
        // inside each row: K >= 8, and N >= 8 for a row-major B
        if (e.sched == 7 && (Kx < 8 || (e.opb == 0 && Nx < 8))) continue;
        if (want_wn && (e.variant == V_MFMA ? e.wn : 1) != want_wn) continue;
        // fp32 tiles that the direct-copy tiles of the same shape dominate where those
        // can run (unless asked for by schedule): the three-stage 64 x 64 tile measured
        // 10-40% slower than the direct-copy one on all 44 shapes timed with both
        // (median 17%), the three-stage and register-staged 256 x 128 tiles within 1-2%
        // of the direct-copy 256 x 128 tile (medians 0.6% and 1.6% slower, at most 4%
        // faster), which leaves their ranking to noise in the fitted times
        if (e.dtype == DT_F32 && e.variant == V_MFMA && !want_sched && (packed || dma_ok) &&
            (e.opb == 1 || Nx % 4 == 0)) {
            if (e.sched == 6 && e.bm == 64 && Kx % 64 == 0 && Kx > 0) continue;
            if ((e.sched == 6 || e.sched == 1) && e.bm == 256 && e.bn == 128 && Kx % 32 == 0 && Kx > 0) continue;
        }
        const int vec = want_vec >= 0 ? want_vec : ((packed || vec_ok) ? 1 : 0);
        if (e.vec != vec) continue;
        if (e.vec && !packed && !vec_ok) continue;          // 16-byte loads need element-aligned bases
        if (direct_copy(e.sched) && !packed && !dma_ok) continue;   // direct LDS copies need 16-byte alignment
        const int64_t tiles = direct_copy(e.sched) ? ((Mx + e.bm - 1) / e.bm) * ((Nx + e.bn - 1) / e.bn)
                                                  : ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
        const int64_t ktiles = (Kx + e.bk - 1) / e.bk;
        const int occ = blocks_per_cu(e);
        const int64_t concurrent = (int64_t)num_cus * occ;
        // A grid capped below the tile count: the persistent form of the
        // software-pipelined direct-copy kernel (whole k-tiles, more than the three
        // its copy stream runs ahead), each workgroup taking one tile per round.
        // Without a cap it is the default where it applies and the tiles outnumber
        // the workgroups the machine holds at once: one workgroup per slot, whose
        // copies of a tile's first k-tiles overlap the previous tile's last ones.
        // Medians of five alternated passes against one workgroup per tile (8 waves,
        // one box): 8192^2 x 512 fp16 85.1 against 96.6 us, 8192^2 x 2048 fp16 238.3
        // against 259.9, 16384 x 8192 x 1024 fp16 288.6 against 327.6, 12288^2 x 512
        // bf16 213.3 against 232.7, 6144^2 x 2048 bf16 151.6 against 156.2, 4608^2 x
        // 1024 fp16 56.7 against 59.3, 4352^2 x 256 fp16 27.1 against 28.8, 8192^3
        // bf16 852.6 against 859.2; with bias, GELU and bf16 output 8192^2 x 1024 fp16
        // 181.2 against 189.5, 8192^2 x 512 bf16 121.3 against 128.1, 8192^2 x 4096
        // 497.0 against 508.8.
        int64_t grid_e = tiles;
        if (want_grid > 0 && tiles > want_grid) {
            if (!persistent_capable(e.sched, e.threads, Kx)) continue;
            grid_e = want_grid;
        } else if (want_grid == 0 && tiles > concurrent && persistent_capable(e.sched, e.threads, Kx)) {
            grid_e = concurrent;
        }
        // split candidates: none, or S slices of whole k-tiles. Three and six slices
        // bring few 256 x 256 tiles near 192 workgroups, where the software-pipelined
        // kernel's split products measured best (medians of three alternated passes,
        // one box: 512 x 4096 x 8192 fp16, 32 tiles, 50.4 us in six slices against 54.1
        // in four and 55.5 in eight; 1024 x 4096 x 4096, 64 tiles, 51.1 in three against
        // 55.2 in two and 54.2 in four)
        const int cand[] = {1, 2, 3, 4, 6, 8, 16};
        // (with stream_k = 2 only the unsplit cost is taken, as the base of the
        // stream-K candidates below, which are then the only ones)
        const int ncand = want_split >= 2 || want_sk == 2 ? 1 : 7;
        double dp_cost_e = -1.0;  // this entry's cost unsplit (the stream-K candidates' base)
        for (int ci = 0; ci < ncand; ++ci) {
            const int S = want_split >= 2 ? want_split : cand[ci];
            if ((want_split == 1 || packed) && S != 1) continue;
            int64_t slices = 1, chunk = Kx;
            if (S > 1) {
                // the register-staged kernels, the one-tile form of the software-
                // pipelined kernels and the fp32 direct-copy tiles take K slices of whole
                // k-tiles (the 64 x 64 direct-copy tile: whole pairs, one per K group)
                if ((e.sched != 1 && e.sched != 5 && e.sched != 7 && e.sched != 8 && e.sched != 9) || ktiles < 2)
                    continue;
                int64_t chunk_tiles = (ktiles + S - 1) / S;
                if (e.sched == 8) chunk_tiles = (chunk_tiles + 1) & ~(int64_t)1;
                slices = (ktiles + chunk_tiles - 1) / chunk_tiles;
                chunk = chunk_tiles * e.bk;
                if (slices < 2) continue;
                // the register-staged software-pipelined kernel reads 16-byte chunks inside
                // its slice: the last slice holds at least 8 k
                if (e.sched == 7 && Kx - (slices - 1) * chunk < 8) continue;
                const int64_t need = split_workspace(slices, M, N);
                if (need > ws_bytes) {
                    if (want_split >= 2) short_ws = std::max(short_ws, need);
                    continue;
                }
            }
            if (grid_e < tiles && S != 1) continue;
            const int64_t work = tiles * slices;
            // persistent: ceil(tiles / grid) tiles per workgroup, the grid in waves of
            // `concurrent` workgroups
            const int64_t rounds = grid_e < tiles ? ((grid_e + concurrent - 1) / concurrent) *
                                                        ((tiles + grid_e - 1) / grid_e)
                                                  : (work + concurrent - 1) / concurrent;
            const int64_t resident =
                std::min<int64_t>(occ, ((grid_e < tiles ? grid_e : work) + num_cus - 1) / num_cus);
            const int64_t kpad = ((std::min<int64_t>(chunk, Kx) + e.bk - 1) / e.bk) * e.bk;
            // The software-pipelined kernel (schedule 5) against the ping-pong kernel and
            // its own 4-wave form, medians of three alternated passes: 8 waves are best or
            // within 1% on both B layouts (column-major B: 4096^3 bf16 113.6 us against
            // 119.1 ping-pong and 118.1 four waves, 8192^3 bf16 862 against 876, 8192^2 x
            // 256 fp16 85.8 against 90.3 and 88.2; row-major B: 8192^2 x 512 fp16 108.2
            // against 116.2 and 115.9, 8192^2 x 256 85.5 against 89.2 and 90.8), except
            // for one round of tiles with at most 32 k-tiles, where the ping-pong kernel
            // is 2-5% faster (4096^2 x 1024 bf16, column-major B: 36.7 against 38.7;
            // 4096^2 x 512 bf16: 25.8 against 26.4). With a fused epilogue (bias, GELU,
            // bf16 out) 8 waves win from 32 k-tiles on, either B layout (column-major B
            // 4096^3 fp16 140.9 against 147.3, bf16 127.1 against 131.0; row-major B
            // 4096^2 x 1024 53.0 against 54.7), the ping-pong kernel at 8 and 16 k-tiles
            // (8192^2 x 256 124.4 against 127.2; 8192^2 x 512 column-major B 150.6
            // against 155.2); 4 waves are 12-60% slower there.
            //
            // The register-staged form (schedule 7) follows the same rules, about 10%
            // slower than the direct copies on the same data (medians of three
            // alternated passes, 8 waves: 4096^3 fp16 134.5 against 123.1 us, 3072 x
            // 5120 x 1088 bf16 41.3 against 40.7); it is the kernel for rows that are
            // not 16-byte aligned: 3001 x 5003 x 1037 bf16 with column-major B 58.3 us
            // against 73 on the register-staged 256 x 256 tile and 62.2 packed, 2000 x
            // 3000 x 1001 fp16 36.4 against 39.2, 4095^3 fp16 156.1 against 161.8 for
            // 4 waves; 8192^2 x 1037 bf16 193.2 against 183.3 packed.
            double eff = tile_efficiency(e, packed || dma_ok);
            if (e.sched == 5 || e.sched == 7) {
                // k-tiles of one workgroup's work (a slice when K is split; the slices'
                // partial products are plain stores, the reduction applies the epilogue)
                const int64_t kt_unit = (std::min<int64_t>(chunk, Kx) + e.bk - 1) / e.bk;
                const bool eight = e.wm * e.wn == 8;
                if (fused_epilogue && slices == 1) eff = eight && ktiles >= 32 ? 0.99 : 0.90;
                else eff = !eight ? 0.90 : (work <= num_cus && kt_unit <= 32) ? 0.96 : 0.99;
                if (e.sched == 7) eff *= 0.9;
            }
            const double tile_cycles = 2.0 * e.bm * e.bn * std::max<int64_t>(kpad, e.bk) / (rate_per_cu(e) * eff);
            double cost = (double)rounds * (double)std::max<int64_t>(resident, 1) * tile_cycles;
            // 16-bit families with a fitted time: the persistent grid measured 2-12%
            // faster than one workgroup per tile over several rounds (0.94 on average),
            // a split adds its reduction (every plane read and C written: 5.5 TB/s
            // fitted on 434 split runs, and 4 us for the second launch, which small
            // problems measured: 768^2 x 512 split four ways 12.1 us against 5.9),
            // packing its copy (3.5 TB/s, plus 3 us for its launch);
            // 16-byte loads from rows that are not 16-byte aligned cost the
            // register-staged kernels 1.8x in the k loop (the load factor above)
            const TimeFit* fit = time_fit(e);
            const int64_t kt_unit = (std::min<int64_t>(chunk, Kx) + e.bk - 1) / e.bk;
            const double flops = 2.0 * (double)Mx * (double)Nx * (double)Kx;
            if (fit && e.dtype == DT_F32) {
                // fp32 tiles with a fitted time; element-wise loads (bases not aligned
                // to the element) are assumed 1.7x slower in the k loop. The split's
                // reduction and the packing copy as below and for 16-bit inputs.
                const double kslow = (!e.vec ? 1.7 : (packed || dma_ok) ? 1.0 : fit->ks) *
                                     (Mx % e.bm != 0 || Nx % e.bn != 0 ? fit->edge : 1.0);
                double t = fit_us(*fit, e, rounds, std::max<int64_t>(resident, 1), kt_unit, flops, kslow);
                if (slices > 1) t += 4.0 + (double)(slices + 1) * (double)M * (double)N * 4.0 / 5.49e6;
                cost = t * kCycles32PerUs + (packed ? pack_cycles : 0.0);
            } else if (fit) {
                const double kslow = e.sched == 1 && !(packed || dma_ok) ? 1.0 / 0.55 : 1.0;
                double t = fit_us(*fit, e, rounds, std::max<int64_t>(resident, 1), kt_unit, flops, kslow);
                if (e.sched == 7 && e.threads != 512) t *= 1.1;
                // where the direct-copy kernels can take the problem (16-byte aligned
                // operands, K a multiple of 8, row-major B with N a multiple of 8), the
                // register-staged software-pipelined form measured about 10% slower
                // than they do (4096^2 x 256 fp16: 21.7 us against 19.4 on the ping-pong
                // kernel)
                if (e.sched == 7 && (packed || dma_ok) && Kx % 8 == 0 && (e.opb == 1 || Nx % 8 == 0)) t *= 1.15;
                // the ping-pong kernel against the 8-wave software-pipelined one, beyond
                // what the fit resolves: past 32 k-tiles 3-16% slower with row-major B
                // (4096^2 x 2048 fp16 70.6 us against 67.3, bf16 67.3 against 62.5;
                // 3072 x 4096 x 2048 62.8 against 53.6), 1% faster with column-major B
                // (67.7 against 68.5); for one full round of at most 32 k-tiles 3-5%
                // faster (4096^2 x 512 fp16 25.8 against 27.0, bf16 25.0 against 26.0;
                // 4096^2 x 1024 39 against 40, bf16 37 against 39); with a fused
                // epilogue the 8-wave kernel is the faster from 32 k-tiles on (4096^2 x
                // 1024, bias, GELU and bf16 out: 53.0 against 54.7)
                if (e.sched == 2) {
                    const bool one_round = rounds == 1 && work * 10 >= (int64_t)num_cus * 9;
                    // (with an epilogue below 32 k-tiles the ping-pong kernel measured
                    // 2-3% faster, 8192^2 x 256 124.4 against 127.2 and 8192^2 x 512
                    // column-major B 150.6 against 155.2, where the fit puts it 10-15%
                    // behind: the factor sets the measured order)
                    if (fused_epilogue) t *= kt_unit < 32 ? 0.85 : 1.03;
                    else if (kt_unit > 32 && e.opb == 0) t *= 1.08;
                    else if (kt_unit <= 16) t *= 0.85;  // 4096^2 x 256 bf16 19.4 against 20.9,
                                                        // 1536 x 8192 x 256 18.2 against 20.4
                    else if (one_round && kt_unit <= 32) t *= 0.95;
                }
                if (grid_e < tiles) t *= 0.94;
                if (slices > 1) t += 4.0 + (double)(slices + 1) * (double)M * (double)N * 4.0 / 5.49e6;
                // K splits of the 8-wave software-pipelined kernel that fill 160 to 256
                // workgroups measured 7-16% under this estimate (a sweep of 13 skinny
                // long-K fp16 problems, 2 to 16 slices each; with the factor the model's
                // choice among the split counts is the measured best on 10 of them, and
                // within 0.5% on average, against 6 and 4.5% without it)
                if (e.sched == 5 && e.threads == 512 && slices > 1 && work >= 160 && work <= num_cus) t *= 0.93;
                if (packed) t += (double)((M * K + K * N) + (Mp * Kp + Np * Kp)) * es / 3.5e6 + 3.0;
                cost = t * kCycles16PerUs;
            } else {
                // the SIMT kernels: the reduction reads every plane and writes C, and is a
                // second launch (about 16000 cycles beyond its traffic at 1 KB per clock)
                if (slices > 1) cost += (double)(slices + 1) * (double)M * (double)N * 4.0 / 1024.0 + 16000.0;
                if (packed) cost += pack_cycles;
            }
            if (slices == 1) dp_cost_e = cost;
            if (want_sk == 2) continue;
            if (!best || cost < best_cost * (1 - 1e-9) ||
                (cost <= best_cost * (1 + 1e-9) && e.bm * e.bn > best->bm * best->bn)) {
                best = &e;
                best_cost = cost;
                best_split = slices;
                best_chunk = chunk;
                best_packed = packed;
                best_grid = grid_e;
                best_sk = 0;
                best_skw = 0;
            }
        }
        // Stream-K tail ("Shared memory and tensor cores" section 13.10) on the
        // persistent software-pipelined kernel: the tiles that leave the last round of
        // a grid of G partly idle (all of them with fewer tiles than G) dealt out as
        // equal k-tile shares to `width` workgroups (more than the tail's tiles, at
        // most G); every share at least 4 k-tiles (whole k-tiles, at least 8 per tile,
        // and S * KT / width >= 4), a 512 KiB workspace slot pair per workgroup, no
        // packing and no split.
        //
        // Cost: this entry's unsplit cost, less the tail's time on one tile per
        // workgroup, plus the tail's time as shares and the fixup. Per k-tile of a
        // 256 x 256 tile, one workgroup takes about 0.42 us while at most ~160 compute
        // units are busy and 0.95 us with all 256 (the chip is power-limited: fewer
        // busy units run at a higher clock); the fixup costs 4 us plus 0.04 us per
        // partial sum (10.6 us for the 165 of 4352^2 x 2048 on 132 workgroups). Fitted on 31 timings (9 shapes, each against its unsplit
        // time, alternated on one box): 4352^2 x 2048 fp16 (tail of 33 tiles of 64
        // k-tiles) 92.6 us on 132 workgroups against 99.5 unsplit; x 8192 279.4
        // against 344.4; x 4096 bf16, column-major B 147.9 against 176.8; 8448 x 8192
        // x 2048 (four rounds and 32 tiles) 272.1 against 278.6; 6144^2 x 2048 bf16
        // (two rounds and 64) 148.9 against 150.2; 4608^2 x 1024 (68 tiles of 32
        // k-tiles) 66.8 against 59.0; 5120^2 x 4096 (144 tiles) 228.9 on 256
        // workgroups against 191.7. A stream-K plan must gain 2% over the unsplit one.
        // The heuristic considers it only behind whole rounds: with fewer tiles than
        // workgroups (all tiles shared) split K is the measured choice (2048^2 x 8192
        // fp16, 64 tiles: 85.3 us in two slices, 82.4-89.4 as stream-K shares on 128
        // to 256 workgroups, which the per-k-tile times above do not model).
        if (want_sk != 1 && !packed && want_split < 2 && e.sched == 5 && e.threads == 512 && Kx % e.bk == 0 &&
            Kx / e.bk >= 8 && dp_cost_e > 0 && (want_sk == 2 || tiles > (want_grid > 0 ? want_grid : concurrent))) {
            const int64_t G = want_grid > 0 ? want_grid : concurrent;
            const int64_t KT = Kx / e.bk;
            const int64_t S = tiles > G ? tiles % G : (tiles < G ? tiles : 0);
            auto kt_us = [&](int64_t busy) {  // one workgroup's time per k-tile
                return busy <= 160 ? 0.42 : 0.42 + 0.53 * (double)(std::min<int64_t>(busy, 256) - 160) / 96.0;
            };
            const double dp_tail = (double)KT * kt_us(S);
            // widths: the one asked for, else 2S, 3S, ... and G
            for (int64_t m = 2; S > 0; ++m) {
                const int64_t width = want_skw > 0 ? want_skw : std::min(m * S, G);
                const bool last = want_skw > 0 || width == G;
                const int64_t need = width * 2 * e.bm * e.bn * 4;
                // (the share arithmetic takes width * S * KT below 2^53)
                const bool fits = width > S && width <= G && (S * KT) / width >= kSkMinPiece &&
                                  (double)width * (double)(S * KT) < 9.0e15;
                if (fits && need > ws_bytes) {
                    if (want_sk == 2) short_ws = short_ws < 0 ? need : std::min(short_ws, need);
                } else if (fits) {
                    const int64_t q = (S * KT + width - 1) / width;
                    const int64_t partials = std::min<int64_t>(2 * width, width + S);
                    const double sk_tail = (double)q * kt_us(width) + 4.0 + 0.04 * (double)partials;
                    const double cost = dp_cost_e * 1.02 + (sk_tail - dp_tail) * kCycles16PerUs;
                    if (!best || cost < best_cost * (1 - 1e-9)) {
                        best = &e;
                        best_cost = cost;
                        best_split = 1;
                        best_chunk = Kx;
                        best_packed = false;
                        best_grid = G;
                        best_sk = S;
                        best_skw = width;
                    }
                }
                if (last) break;
            }
        }
    }
    }
    if (!best && want_sk == 2 && short_ws > 0) {
        set_error("stream_k = 2 needs at least %lld bytes of workspace; %lld were given", (long long)short_ws,
                  (long long)ws_bytes);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (!best && want_sk == 2) {
        set_error("stream_k = 2 does not apply: it needs the 8-wave schedule-5 kernel (16-bit inputs, 16-byte aligned "
                  "operands), K a multiple of 32 with at least 8 k-tiles, no packing or split, a tile count that "
                  "leaves a partial round of the grid, shares of at least 4 k-tiles and sk_width above the tail's tiles "
                  "and at most the grid");
        return GEMM_ERR_INVALID_VALUE;
    }
    if (!best && short_ws > 0) {
        set_error("split_k = %d needs %lld bytes of workspace; %lld were given", want_split, (long long)short_ws,
                  (long long)ws_bytes);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (!best) {
        set_error("no compiled kernel matches: dtype %s, opB %s, variant %d, bm %d, bn %d, vec %d%s",
                  dtype_name(dtype), opB == GEMM_OP_N ? "N" : "T", want_variant, want_bm, want_bn, want_vec,
                  want_grid > 0 ? " (a max_grid below the tile count needs the 8-wave schedule-5 kernel: 16-byte "
                                  "aligned operands or packing, K a multiple of 32 and at least 128, no split)"
                                : "");
        return GEMM_ERR_UNSUPPORTED;
    }
    const MenuEntry& e = *best;
    gemm_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.variant = e.variant;
    cfg.bm = e.bm;
    cfg.bn = e.bn;
    cfg.bk = e.bk;
    cfg.vec = e.vec;
    cfg.waves_m = e.variant == V_MFMA ? e.wm : 1;
    cfg.waves_n = e.variant == V_MFMA ? e.wn : 1;
    cfg.thread_m = e.tm;
    cfg.thread_n = e.tn;
    cfg.threads = e.threads;
    cfg.lds_bytes = e.lds_bytes;
    cfg.kernel_id = e.id;
    cfg.schedule = e.sched;
    cfg.tiles_m = ((best_packed && direct_copy(e.sched) ? Mp : M) + e.bm - 1) / e.bm;
    cfg.tiles_n = ((best_packed && direct_copy(e.sched) ? Np : N) + e.bn - 1) / e.bn;
    cfg.grid = (int32_t)(best_sk > 0 ? best_grid : std::min<int64_t>(cfg.tiles_m * cfg.tiles_n, best_grid));
    cfg.max_grid = want_grid;
    // Group enough tile rows that one XCD's share of the grid forms a compact
    // rectangle; the remap needs the grid to split evenly over the 8 XCDs.
    const int gm = want_group ? want_group : default_group_m(cfg.tiles_m, cfg.tiles_n);
    cfg.group_m = (int32_t)std::max<int64_t>(1, std::min<int64_t>(gm, cfg.tiles_m));
    cfg.tiles_total = cfg.tiles_m * cfg.tiles_n;
    cfg.launches = (best_split > 1 || best_packed || best_sk > 0) ? 2 : 1;
    cfg.stream_k = best_sk > 0 ? 2 : 1;
    cfg.sk_width = (int32_t)best_skw;
    cfg.split_k = (int32_t)best_split;
    cfg.k_chunk = (int32_t)best_chunk;
    cfg.pack = best_packed ? 2 : 1;
    cfg.workspace_bytes = best_split > 1    ? split_workspace(best_split, M, N)
                          : best_packed     ? pack_need
                          : best_sk > 0     ? best_skw * 2 * (int64_t)e.bm * e.bn * 4
                                            : 0;
    cfg.xcd_remap = want_remap >= 0 ? want_remap : ((cfg.grid % 8 == 0 && cfg.grid >= 16) ? 1 : 0);
    cfg.est_cycles = best_cost;
    *out = cfg;
    return GEMM_OK;
}

// ---- plan cache. A plan depends on the problem (operand flags, sizes, leading
// dimensions, dtype), on A's and B's addresses only through their offsets mod 16,
// on the device (CU count, architecture), the workspace size, whether an epilogue
// is fused, and the request's input fields. Successful plans are kept in a small
// direct-mapped table keyed on exactly those, so that a repeated call skips the
// cost model (a few microseconds of host time, as much as a small product takes on
// the device). Failed plans are not kept: each failure sets its message anew.
namespace {

struct PlanKey {
    int64_t M, N, K, lda, ldb, ldc, ws;
    int32_t opA, opB, dtype, num_cus, a16, b16, fused, has_req;
    int32_t req[15];
    char arch[32];
};

struct PlanSlot {
    bool used;
    PlanKey key;
    gemm_config cfg;
};

constexpr int kPlanSlots = 256;
std::mutex g_plan_mutex;
PlanSlot g_plan_cache[kPlanSlots];

bool make_key(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
              uintptr_t a, uintptr_t b, int num_cus, const char* arch, int64_t ws_bytes, bool fused,
              const gemm_config* req, PlanKey* k) {
    if (arch == nullptr || strlen(arch) >= sizeof k->arch) return false;
    memset(k, 0, sizeof *k);  // padding included, so that keys compare with memcmp
    k->M = M;
    k->N = N;
    k->K = K;
    k->lda = lda;
    k->ldb = ldb;
    k->ldc = ldc;
    k->ws = ws_bytes;
    k->opA = opA;
    k->opB = opB;
    k->dtype = dtype;
    k->num_cus = num_cus;
    k->a16 = (int32_t)(a & 15);
    k->b16 = (int32_t)(b & 15);
    k->fused = fused ? 1 : 0;
    k->has_req = req != nullptr;
    if (req) {
        const int32_t in[15] = {req->variant, req->bm,       req->bn,      req->vec,     req->xcd_remap,
                                req->group_m, req->waves_m,  req->waves_n, req->schedule, req->max_grid,
                                req->split_k, req->pack,     req->threads, req->stream_k, req->sk_width};
        memcpy(k->req, in, sizeof in);
    }
    memcpy(k->arch, arch, strlen(arch));
    return true;
}

uint32_t key_hash(const PlanKey& k) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(&k);
    uint32_t h = 2166136261u;  // FNV-1a
    for (size_t i = 0; i < sizeof k; ++i) h = (h ^ p[i]) * 16777619u;
    return h;
}

}  // namespace

int plan(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
         uintptr_t a, uintptr_t b, uintptr_t c, int num_cus, const char* arch, int64_t ws_bytes,
         bool fused_epilogue, const gemm_config* req, gemm_config* out) {
    (void)c;
    PlanKey key;
    const bool cacheable = make_key(opA, opB, M, N, K, lda, ldb, ldc, dtype, a, b, num_cus, arch, ws_bytes,
                                    fused_epilogue, req, &key);
    const uint32_t slot = cacheable ? key_hash(key) % kPlanSlots : 0;
    if (cacheable) {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        const PlanSlot& e = g_plan_cache[slot];
        if (e.used && memcmp(&e.key, &key, sizeof key) == 0) {
            *out = e.cfg;
            return GEMM_OK;
        }
    }
    const int st = plan_uncached(opA, opB, M, N, K, lda, ldb, ldc, dtype, a, b, num_cus, arch, ws_bytes,
                                 fused_epilogue, req, out);
    if (st == GEMM_OK && cacheable) {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        PlanSlot& e = g_plan_cache[slot];
        e.used = true;
        e.key = key;
        e.cfg = *out;
    }
    return st;
}

int default_group_m(int64_t tiles_m, int64_t tiles_n) {
    const int64_t per_xcd = std::max<int64_t>(1, tiles_m * tiles_n / 8);
    int gm = 1;
    while ((int64_t)gm * gm * 2 < per_xcd && gm < tiles_m) gm *= 2;
    return gm;
}

int validate_problem(int opA, int opB, int dtype, const gemm_problem& p, int index) {
    int st = validate(opA, opB, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, dtype);
    if (st != GEMM_OK) {
        const std::string why = g_last_error;
        set_error("problem %d: %s", index, why.c_str());
        return st;
    }
    if (p.batch < 0 || p.stride_a < 0 || p.stride_b < 0 || p.stride_c < 0) {
        set_error("problem %d: batch (%lld) and strides (%lld, %lld, %lld) must be non-negative", index,
                  (long long)p.batch, (long long)p.stride_a, (long long)p.stride_b, (long long)p.stride_c);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (p.ldc >= ((int64_t)1 << 31)) {
        set_error("problem %d: ldc = %lld must be below 2^31 in a grouped call", index, (long long)p.ldc);
        return GEMM_ERR_UNSUPPORTED;
    }
    if (p.batch > 1 && p.M > 0 && p.N > 0 && p.stride_c < (p.M - 1) * p.ldc + p.N) {
        set_error("problem %d: stride_c = %lld is smaller than one output, (M-1)*ldc + N = %lld, so the batch's "
                  "outputs would overlap", index, (long long)p.stride_c, (long long)((p.M - 1) * p.ldc + p.N));
        return GEMM_ERR_INVALID_VALUE;
    }
    return GEMM_OK;
}

// Grouped heuristic: the same cost model as plan(), with the work of every
// problem spread over the compute units the persistent grid occupies; a tile is
// never split, so the longest tile bounds the estimate from below.
int plan_grouped(int opA, int opB, int dtype, const gemm_problem* probs, int count, int num_cus, const char* arch,
                 const gemm_config* req, gemm_config* out) {
    if (count < 0) {
        set_error("count = %d must be non-negative", count);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (count > 0 && probs == nullptr) {
        set_error("problems is NULL with count = %d", count);
        return GEMM_ERR_NULL_POINTER;
    }
    for (int i = 0; i < count; ++i) {
        const int st = validate_problem(opA, opB, dtype, probs[i], i);
        if (st != GEMM_OK) return st;
    }
    if (arch == nullptr || strncmp(arch, "gfx950", 6) != 0) {
        set_error("device architecture '%s' is not gfx950; the kernels are built for gfx950 only",
                  arch ? arch : "(null)");
        return GEMM_ERR_DEVICE;
    }
    if (num_cus <= 0) {
        set_error("compute-unit count %d must be positive", num_cus);
        return GEMM_ERR_INVALID_VALUE;
    }
    const int es = elem_size(dtype);
    bool vec_ok = true, rows16 = true, sp_ok = dtype != GEMM_F32;
    for (int i = 0; i < count; ++i) {
        const gemm_problem& p = probs[i];
        if (p.M == 0 || p.N == 0 || p.batch == 0) continue;
        // the persistent software-pipelined form: whole k-tiles of 32, at least four
        // (its copy stream runs three ahead across tiles), row-major B in chunks of 8
        sp_ok = sp_ok && p.K % 32 == 0 && p.K / 32 > 3 && (opB == GEMM_OP_T || p.N % 8 == 0);
        // batch strides are in elements, so every batch stays element-aligned
        vec_ok = vec_ok && elem_aligned((uintptr_t)p.A, es) && elem_aligned((uintptr_t)p.B, es);
        rows16 = rows16 && aligned16((uintptr_t)p.A) && aligned16((uintptr_t)p.B) && (p.lda * es) % 16 == 0 &&
                 (p.ldb * es) % 16 == 0 &&
                 (p.batch <= 1 || ((p.stride_a * es) % 16 == 0 && (p.stride_b * es) % 16 == 0));
    }
    int want_variant = GEMM_VARIANT_AUTO, want_bm = 0, want_bn = 0, want_vec = -1, want_remap = -1, want_group = 0;
    int want_wm = 0, want_wn = 0, want_sched = 0, want_grid = 0, want_threads = 0;
    if (req) {
        want_variant = req->variant;
        want_bm = req->bm;
        want_bn = req->bn;
        want_vec = req->vec;
        want_remap = req->xcd_remap;
        want_group = req->group_m;
        want_wm = req->waves_m;
        want_wn = req->waves_n;
        want_sched = req->schedule;
        want_grid = req->max_grid;
        want_threads = req->threads;
        if (want_variant < 0 || want_variant > 2 || want_vec < -1 || want_vec > 1 || want_remap < -1 || want_remap > 1 ||
            want_group < 0 || want_bm < 0 || want_bn < 0 || want_wm < 0 || want_wn < 0 || want_sched < 0 ||
            want_grid < 0 || want_threads < 0) {
            set_error("invalid requested configuration (variant %d, bm %d, bn %d, vec %d, xcd_remap %d, group_m %d, "
                      "max_grid %d)", want_variant, want_bm, want_bn, want_vec, want_remap, want_group, want_grid);
            return GEMM_ERR_INVALID_VALUE;
        }
        if (want_sched > 1 && want_sched != 5) {
            set_error("schedule %d has no grouped form; grouped calls run the register-staged schedule (1) or "
                      "the persistent software-pipelined one (5)", want_sched);
            return GEMM_ERR_UNSUPPORTED;
        }
        if (req->split_k > 1 || req->pack == 2) {
            set_error("grouped calls neither split K nor pack operands (split_k = %d, pack = %d)", req->split_k,
                      req->pack);
            return GEMM_ERR_UNSUPPORTED;
        }
        if (want_vec == 1 && !vec_ok) {
            set_error("16-byte loads requested but some A/B base is not aligned to the element size");
            return GEMM_ERR_UNSUPPORTED;
        }
    }
    const MenuEntry* best = nullptr;
    double best_cost = 0;
    int64_t best_tiles = 0, best_grid = 0;
    for (const MenuEntry& e : kMenu) {
        if (e.dtype != dtype || e.opb != opB) continue;
        if (!grouped_capable(e.variant, e.sched, e.bm, e.bn, e.wm, e.wn, e.threads)) continue;
        if (e.sched == 5 && !(sp_ok && rows16)) continue;
        if (want_sched && e.sched != want_sched) continue;
        if (want_threads && e.threads != want_threads) continue;
        if (want_variant != GEMM_VARIANT_AUTO && e.variant != want_variant) continue;
        if (want_bm && e.bm != want_bm) continue;
        if (want_bn && e.bn != want_bn) continue;
        if (want_wm && (e.variant == V_MFMA ? e.wm : 1) != want_wm) continue;
        if (want_wn && (e.variant == V_MFMA ? e.wn : 1) != want_wn) continue;
        const int vec = want_vec >= 0 ? want_vec : (vec_ok ? 1 : 0);
        if (e.vec != vec) continue;
        int64_t tiles = 0;
        double work = 0, longest = 0;
        for (int i = 0; i < count; ++i) {
            const gemm_problem& p = probs[i];
            if (p.M == 0 || p.N == 0 || p.batch == 0) continue;
            const int64_t t = p.batch * ((p.M + e.bm - 1) / e.bm) * ((p.N + e.bn - 1) / e.bn);
            const int64_t kpad = std::max<int64_t>(((p.K + e.bk - 1) / e.bk) * e.bk, e.bk);
            // the persistent software-pipelined form streams its copies across tiles
            // and problems; strided batches against the register-staged grouped kernel,
            // medians of five alternated passes: 4 x 4096^2 x 1024 bf16 147.9 us against
            // 165.1 (and 155.3 as four calls), 8 x 2048^3 bf16 127.3 against 144.5,
            // 32 x 1024^3 bf16 74.5 against 91.8, 16 x 1024^2 x 512 fp16 28.0 against
            // 31.8, 64 x 512^3 fp16 31.8 against 32.6
            const double eff = e.sched == 5 ? 0.99 : tile_efficiency(e, rows16);
            const double tc = 2.0 * e.bm * e.bn * (double)kpad / (rate_per_cu(e) * eff);
            tiles += t;
            work += (double)t * tc;
            longest = std::max(longest, tc);
        }
        int64_t grid = std::min<int64_t>(tiles, (int64_t)num_cus * blocks_per_cu(e));
        if (want_grid) grid = std::min<int64_t>(grid, want_grid);
        const double cost = tiles == 0 ? 0 : std::max(work / (double)std::min<int64_t>(grid, num_cus), longest);
        if (!best || cost < best_cost * (1 - 1e-9) ||
            (cost <= best_cost * (1 + 1e-9) && e.bm * e.bn > best->bm * best->bn)) {
            best = &e;
            best_cost = cost;
            best_tiles = tiles;
            best_grid = grid;
        }
    }
    if (!best) {
        set_error("no compiled grouped kernel matches: dtype %s, opB %s, variant %d, bm %d, bn %d, vec %d",
                  dtype_name(dtype), opB == GEMM_OP_N ? "N" : "T", want_variant, want_bm, want_bn, want_vec);
        return GEMM_ERR_UNSUPPORTED;
    }
    // linear tile indices and the persistent loop's t + grid stay below 2^31
    if (best_tiles >= ((int64_t)1 << 31) - ((int64_t)1 << 16)) {
        set_error("%lld output tiles in one grouped call; at most 2^31 - 2^16 are supported", (long long)best_tiles);
        return GEMM_ERR_UNSUPPORTED;
    }
    const MenuEntry& e = *best;
    gemm_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.variant = e.variant;
    cfg.bm = e.bm;
    cfg.bn = e.bn;
    cfg.bk = e.bk;
    cfg.vec = e.vec;
    cfg.waves_m = e.variant == V_MFMA ? e.wm : 1;
    cfg.waves_n = e.variant == V_MFMA ? e.wn : 1;
    cfg.thread_m = e.tm;
    cfg.thread_n = e.tn;
    cfg.threads = e.threads;
    cfg.lds_bytes = e.lds_bytes;
    cfg.kernel_id = e.id;
    cfg.schedule = e.sched;
    int segments = 0;
    for (int i = 0; i < count; ++i) {
        const gemm_problem& p = probs[i];
        if (p.M == 0 || p.N == 0 || p.batch == 0) continue;
        if (segments == 0) {
            cfg.tiles_m = (p.M + e.bm - 1) / e.bm;
            cfg.tiles_n = (p.N + e.bn - 1) / e.bn;
        }
        ++segments;
    }
    cfg.group_m = want_group;  // 0: per problem, default_group_m
    cfg.grid = (int32_t)best_grid;
    cfg.max_grid = want_grid;
    cfg.xcd_remap = want_remap >= 0 ? want_remap : ((cfg.grid % 8 == 0 && cfg.grid >= 16) ? 1 : 0);
    cfg.tiles_total = best_tiles;
    cfg.launches = (segments + kMaxGroupSegments - 1) / kMaxGroupSegments;
    cfg.split_k = 1;
    cfg.pack = 1;
    cfg.est_cycles = best_cost;
    *out = cfg;
    return GEMM_OK;
}

int menu_entry(int index, int* variant, int* dtype, int* opb, gemm_config* out) {
    if (index < 0 || index >= kMenuSize) {
        set_error("menu index %d out of range [0, %d)", index, kMenuSize);
        return GEMM_ERR_INVALID_VALUE;
    }
    const MenuEntry& e = kMenu[index];
    if (variant) *variant = e.variant;
    if (dtype) *dtype = e.dtype;
    if (opb) *opb = e.opb;
    if (out) {
        memset(out, 0, sizeof *out);
        out->variant = e.variant;
        out->bm = e.bm;
        out->bn = e.bn;
        out->bk = e.bk;
        out->vec = e.vec;
        out->waves_m = e.variant == V_MFMA ? e.wm : 1;
        out->waves_n = e.variant == V_MFMA ? e.wn : 1;
        out->thread_m = e.tm;
        out->thread_n = e.tn;
        out->threads = e.threads;
        out->lds_bytes = e.lds_bytes;
        out->kernel_id = e.id;
        out->schedule = e.sched;
        out->xcd_remap = -1;
    }
    return GEMM_OK;
}

}  // namespace dg
