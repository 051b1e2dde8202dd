// menu.h -- the compiled kernel configurations and the launch-argument block.
//
// Internal to the library. Host-only code (the planner) reads the menu as plain
// data; the HIP translation units instantiate one kernel per entry. Keeping the
// list in one X-macro is what keeps the two sides consistent.
#pragma once
#include <stdint.h>

namespace dg {

enum Variant { V_LDS = 1, V_MFMA = 2 };
enum Dtype { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// One kernel configuration.
//   variant : V_LDS (LDS-staged SIMT FMA) or V_MFMA (matrix cores)
//   dtype   : input element type (accumulation and C are fp32)
//   opb     : 0 = B row-major K x N, 1 = B column-major (row-major N x K)
//   vec     : 1 = 16-byte global loads (needs aligned bases and leading dims),
//             0 = element-wise loads (any alignment)
//   bm, bn, bk : block tile; wm x wn : wave grid (MFMA); tm x tn : thread tile (LDS)
//   sched   : 1 = register-staged double buffer (any shape), 2 = ping-pong with
//             direct global->LDS copies on 16x16x32 MFMAs, 3 = not used (an earlier
//             kernel, removed), 4 = ping-pong on 32x32x16 MFMAs, 5 = software-
//             pipelined 32x32x16 with direct copies, 4 waves of 128 x 128 or 8 of
//             128 x 64 (2, 4, 5: 16-byte aligned operands, edge tiles in M, and in N
//             for column-major B or N a multiple of 8; 2, 4: K a multiple of bk;
//             5: K a multiple of 8), 6 = register-staged with three LDS stages and fragments
//             read a half k-tile ahead (fp32, any shape), 7 = the software-pipelined
//             32x32x16 kernel of schedule 5 with register-staged loads (16-bit inputs,
//             bases aligned to the element, any M, K >= 8, N >= 8 for row-major B),
//             8 = fp32 64 x 64 tiles with direct copies three k-tiles ahead (16-byte
//             aligned operands, K a multiple of 64, N a multiple of 4 for row-major B),
//             9 = fp32 256 x 128 and 128 x 128 tiles on eight waves with direct copies
//             two (three LDS stages) or three (four) k-tiles ahead (16-byte aligned
//             operands, K a multiple of 32, N a multiple of 4 for row-major B)
struct MenuEntry {
    int id, variant, dtype, opb, vec, bm, bn, bk, wm, wn, tm, tn, threads, lds_bytes, sched;
};

// Schedules the planner may choose and the launcher will run. Schedule 3 (a
// software-pipelined kernel whose copies were issued from inline assembly) faulted
// on the device and was removed from the library; the number stays unused so that
// configurations keep their meaning, and requests for it are refused.
constexpr bool schedule_enabled(int sched) { return sched != 3; }

// Schedules whose kernels copy tiles straight into LDS: the operands must be 16-byte
// aligned and K whole k-tiles (schedule 5: K a multiple of 8, a partial last k-tile
// zeroed past K); edge tiles in M and N copy clamped rows and columns.
constexpr bool direct_copy(int sched) {
    return sched == 2 || sched == 4 || sched == 5 || sched == 8 || sched == 9;
}

// Configurations with a persistent single-problem form (a grid below the tile count,
// each workgroup striding through the tiles): the 8-wave software-pipelined
// direct-copy kernel, with K (padded K when packed) whole k-tiles of 32, more than
// three of them. (The 4-wave form's 256 accumulators do not stay in registers
// across its tile loop.)
constexpr bool persistent_capable(int sched, int threads, int64_t K) {
    return sched == 5 && threads == 512 && K % 32 == 0 && K / 32 > 3;
}

// Shortest piece of a stream-K share, in k-tiles: the copy distance of the
// persistent kernel plus one (streamk.h).
constexpr int kSkMinPiece = 4;

// Configurations whose kernel applies a fused epilogue (every other one stores the
// plain fp32 accumulator only): all but the 32x32x16 ping-pong kernel.
constexpr bool epilogue_capable(int sched) { return sched != 4; }

// Configurations that also have a grouped (persistent) form: the register-staged
// schedule, which masks every edge, except the 4-wave 256 x 256 tiles (their
// grouped form runs out of registers) and the MFMA tiles that split K between wave
// groups (threads = KG x 64 x wm x wn); and the 8-wave software-pipelined
// direct-copy kernel on its persistent form (every problem 16-byte aligned with K a
// multiple of 32 and at least 128, row-major B with N a multiple of 8).
constexpr bool grouped_capable(int variant, int sched, int bm, int bn, int wm, int wn, int threads) {
    return (sched == 1 && !(bm == 256 && bn == 256 && wm * wn == 4) &&
            (variant != V_MFMA || threads == wm * wn * 64)) ||
           (sched == 5 && threads == 512);
}

// X(id, variant, dtype, opb, vec, bm, bn, bk, wm, wn, tm, tn, threads, lds_bytes, sched)
// The largest MFMA tile is 256 x 256 (2 x 4 waves) for 16-bit inputs and 256 x 128
// (4 x 2 waves) for fp32; the fp32 kernel's 64 x 64 tile uses a 4 x 1 wave grid
// (its row-major-B path needs 64-wide wave tiles).
// LDS bytes: LDS variant holds two fp32 stages of A^T (bk x bm) and B (bk x bn);
// MFMA variant holds two stages of the input-typed A (bm x bk) and B (bk x bn).
#define DG_LDS_ENTRIES(X, base, dt, bk)                                                  \
    X(base + 0, V_LDS, dt, 0, 1, 128, 128, bk, 1, 1, 8, 8, 256, 2 * 4 * bk * 256, 1)          \
    X(base + 1, V_LDS, dt, 1, 1, 128, 128, bk, 1, 1, 8, 8, 256, 2 * 4 * bk * 256, 1)          \
    X(base + 2, V_LDS, dt, 0, 0, 128, 128, bk, 1, 1, 8, 8, 256, 2 * 4 * bk * 256, 1)          \
    X(base + 3, V_LDS, dt, 1, 0, 128, 128, bk, 1, 1, 8, 8, 256, 2 * 4 * bk * 256, 1)          \
    X(base + 4, V_LDS, dt, 0, 1, 64, 64, bk, 1, 1, 4, 4, 256, 2 * 4 * bk * 128, 1)            \
    X(base + 5, V_LDS, dt, 1, 1, 64, 64, bk, 1, 1, 4, 4, 256, 2 * 4 * bk * 128, 1)            \
    X(base + 6, V_LDS, dt, 0, 0, 64, 64, bk, 1, 1, 4, 4, 256, 2 * 4 * bk * 128, 1)            \
    X(base + 7, V_LDS, dt, 1, 0, 64, 64, bk, 1, 1, 4, 4, 256, 2 * 4 * bk * 128, 1)

#define DG_MFMA_ENTRIES(X, base, dt, es, bk, BBM, BBN, BWM, BWN, w64m, w64n)                            \
    X(base + 0, V_MFMA, dt, 0, 1, BBM, BBN, bk, BWM, BWN, 0, 0, 512, 2 * es * bk * (BBM + BBN), 1) \
    X(base + 1, V_MFMA, dt, 1, 1, BBM, BBN, bk, BWM, BWN, 0, 0, 512, 2 * es * bk * (BBM + BBN), 1) \
    X(base + 2, V_MFMA, dt, 0, 0, BBM, BBN, bk, BWM, BWN, 0, 0, 512, 2 * es * bk * (BBM + BBN), 1) \
    X(base + 3, V_MFMA, dt, 1, 0, BBM, BBN, bk, BWM, BWN, 0, 0, 512, 2 * es * bk * (BBM + BBN), 1) \
    X(base + 4, V_MFMA, dt, 0, 1, 128, 128, bk, 2, 2, 0, 0, 256, 2 * es * bk * 256, 1)        \
    X(base + 5, V_MFMA, dt, 1, 1, 128, 128, bk, 2, 2, 0, 0, 256, 2 * es * bk * 256, 1)        \
    X(base + 6, V_MFMA, dt, 0, 0, 128, 128, bk, 2, 2, 0, 0, 256, 2 * es * bk * 256, 1)        \
    X(base + 7, V_MFMA, dt, 1, 0, 128, 128, bk, 2, 2, 0, 0, 256, 2 * es * bk * 256, 1)        \
    X(base + 8, V_MFMA, dt, 0, 1, 64, 64, bk, w64m, w64n, 0, 0, 256, 2 * es * bk * 128, 1)    \
    X(base + 9, V_MFMA, dt, 1, 1, 64, 64, bk, w64m, w64n, 0, 0, 256, 2 * es * bk * 128, 1)    \
    X(base + 10, V_MFMA, dt, 0, 0, 64, 64, bk, w64m, w64n, 0, 0, 256, 2 * es * bk * 128, 1)   \
    X(base + 11, V_MFMA, dt, 1, 0, 64, 64, bk, w64m, w64n, 0, 0, 256, 2 * es * bk * 128, 1)

// 16-bit 256 x 256 tiles with 4 waves of 128 x 128 (one wave per SIMD, accumulators in
// the accumulation registers): half the LDS reads per FLOP of the 8-wave layout.
#define DG_MFMA_WIDE(X, base, dt)                                                        \
    X(base + 0, V_MFMA, dt, 0, 1, 256, 256, 64, 2, 2, 0, 0, 256, 2 * 2 * 64 * 512, 1)         \
    X(base + 1, V_MFMA, dt, 1, 1, 256, 256, 64, 2, 2, 0, 0, 256, 2 * 2 * 64 * 512, 1)         \
    X(base + 2, V_MFMA, dt, 0, 0, 256, 256, 64, 2, 2, 0, 0, 256, 2 * 2 * 64 * 512, 1)         \
    X(base + 3, V_MFMA, dt, 1, 0, 256, 256, 64, 2, 2, 0, 0, 256, 2 * 2 * 64 * 512, 1)

// Ping-pong kernels (16-bit inputs, full 256 x 256 tiles, 4 LDS stages of k = 32).
#define DG_MFMA_PP(X, base, dt)                                                          \
    X(base + 0, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 2)      \
    X(base + 1, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 2)

// The same ping-pong schedule on v_mfma_f32_32x32x16 (half the MFMA instructions).
#define DG_MFMA_PP32(X, base, dt)                                                        \
    X(base + 0, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 4)      \
    X(base + 1, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 4)

// Software-pipelined kernels (16-bit inputs, full tiles, 4 LDS stages of k = 32,
// 32x32x16 MFMAs): 4 waves of 128 x 128 and 8 waves of 128 x 64.
#define DG_MFMA_SP(X, base, dt)                                                          \
    X(base + 0, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 2, 0, 0, 256, 4 * 2 * 32 * 512, 5)      \
    X(base + 1, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 2, 0, 0, 256, 4 * 2 * 32 * 512, 5)      \
    X(base + 2, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 5)      \
    X(base + 3, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 5)

// The software-pipelined kernels with register-staged loads (schedule 7): 16-byte
// loads from element-aligned rows, so no alignment or divisibility beyond K >= 8 (and
// N >= 8 for row-major B).
#define DG_MFMA_SPR(X, base, dt)                                                         \
    X(base + 0, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 2, 0, 0, 256, 4 * 2 * 32 * 512, 7)      \
    X(base + 1, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 2, 0, 0, 256, 4 * 2 * 32 * 512, 7)      \
    X(base + 2, V_MFMA, dt, 0, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 7)      \
    X(base + 3, V_MFMA, dt, 1, 1, 256, 256, 32, 2, 4, 0, 0, 512, 4 * 2 * 32 * 512, 7)

// fp32 64 x 64 tiles with K split between two groups of 4 waves inside the
// workgroup (8 waves: two per SIMD for a tile that holds four); LDS: two stages
// per group.
#define DG_MFMA_KG2(X, base)                                                             \
    X(base + 0, V_MFMA, DT_F32, 0, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 2 * 4 * 32 * 128, 1)   \
    X(base + 1, V_MFMA, DT_F32, 1, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 2 * 4 * 32 * 128, 1)   \
    X(base + 2, V_MFMA, DT_F32, 0, 0, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 2 * 4 * 32 * 128, 1)   \
    X(base + 3, V_MFMA, DT_F32, 1, 0, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 2 * 4 * 32 * 128, 1)

// fp32 256 x 128 tiles on the three-stage schedule (6): LDS holds three stages.
#define DG_MFMA_F32S3(X, base)                                                           \
    X(base + 0, V_MFMA, DT_F32, 0, 1, 256, 128, 32, 4, 2, 0, 0, 512, 3 * 4 * 32 * 384, 6)     \
    X(base + 1, V_MFMA, DT_F32, 1, 1, 256, 128, 32, 4, 2, 0, 0, 512, 3 * 4 * 32 * 384, 6)

// Small fp32 tiles. 16 x 64 with K split over four groups of one wave (256 threads,
// two LDS stages per group): 64 workgroups at 256^3, where 64 x 64 tiles give 16.
// 64 x 64 with K split over two groups of four waves on the three-stage schedule
// (6): the next k-tile's fragments read before the barrier, copies two k-tiles
// ahead.
#define DG_MFMA_F32SMALL(X, base)                                                        \
    X(base + 0, V_MFMA, DT_F32, 0, 1, 16, 64, 32, 1, 1, 0, 0, 256, 4 * 2 * 4 * 32 * 80, 1)     \
    X(base + 1, V_MFMA, DT_F32, 1, 1, 16, 64, 32, 1, 1, 0, 0, 256, 4 * 2 * 4 * 32 * 80, 1)     \
    X(base + 2, V_MFMA, DT_F32, 0, 0, 16, 64, 32, 1, 1, 0, 0, 256, 4 * 2 * 4 * 32 * 80, 1)     \
    X(base + 3, V_MFMA, DT_F32, 1, 0, 16, 64, 32, 1, 1, 0, 0, 256, 4 * 2 * 4 * 32 * 80, 1)     \
    X(base + 4, V_MFMA, DT_F32, 0, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 3 * 4 * 32 * 128, 6)    \
    X(base + 5, V_MFMA, DT_F32, 1, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 3 * 4 * 32 * 128, 6)

// fp32 64 x 64 tiles with direct copies (schedule 8): two K groups of four waves,
// four LDS stages per group (16-byte aligned operands, K a multiple of 64, row-major
// B with N a multiple of 4).
#define DG_MFMA_F32DC(X, base)                                                           \
    X(base + 0, V_MFMA, DT_F32, 0, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 4 * 2 * 8192, 8)        \
    X(base + 1, V_MFMA, DT_F32, 1, 1, 64, 64, 32, 4, 1, 0, 0, 512, 2 * 4 * 2 * 8192, 8)

// fp32 tiles with direct copies on eight waves (schedule 9): 256 x 128 (4 x 2 waves of
// 64 x 64, three LDS stages of 48 KB) and 128 x 128 (4 x 2 waves of 32 x 64, four
// stages of 32 KB).
#define DG_MFMA_F32DCL(X, base)                                                          \
    X(base + 0, V_MFMA, DT_F32, 0, 1, 256, 128, 32, 4, 2, 0, 0, 512, 3 * 4 * 32 * 384, 9)     \
    X(base + 1, V_MFMA, DT_F32, 1, 1, 256, 128, 32, 4, 2, 0, 0, 512, 3 * 4 * 32 * 384, 9)     \
    X(base + 2, V_MFMA, DT_F32, 0, 1, 128, 128, 32, 4, 2, 0, 0, 512, 5 * 4 * 32 * 256, 9)     \
    X(base + 3, V_MFMA, DT_F32, 1, 1, 128, 128, 32, 4, 2, 0, 0, 512, 5 * 4 * 32 * 256, 9)

#define DG_MENU(X)                                              \
    DG_LDS_ENTRIES(X, 0, DT_F32, 16)            \
    DG_LDS_ENTRIES(X, 8, DT_F16, 32)            \
    DG_LDS_ENTRIES(X, 16, DT_BF16, 32)          \
    DG_MFMA_ENTRIES(X, 24, DT_F32, 4, 32, 256, 128, 4, 2, 4, 1) \
    DG_MFMA_ENTRIES(X, 36, DT_F16, 2, 64, 256, 256, 2, 4, 2, 2) \
    DG_MFMA_ENTRIES(X, 48, DT_BF16, 2, 64, 256, 256, 2, 4, 2, 2) \
    DG_MFMA_WIDE(X, 60, DT_F16)                                  \
    DG_MFMA_WIDE(X, 64, DT_BF16)                                 \
    DG_MFMA_PP(X, 68, DT_F16)                                    \
    DG_MFMA_PP(X, 70, DT_BF16)                                   \
    DG_MFMA_PP32(X, 72, DT_F16)                                  \
    DG_MFMA_PP32(X, 74, DT_BF16)                                 \
    DG_MFMA_SP(X, 76, DT_F16)                                    \
    DG_MFMA_SP(X, 80, DT_BF16)                                   \
    DG_MFMA_KG2(X, 84)                                           \
    DG_MFMA_F32S3(X, 88)                                         \
    DG_MFMA_SPR(X, 90, DT_F16)                                   \
    DG_MFMA_SPR(X, 94, DT_BF16)                                  \
    DG_MFMA_F32SMALL(X, 98)                                      \
    DG_MFMA_F32DC(X, 104)                                        \
    DG_MFMA_F32DCL(X, 106)

constexpr int kMenuSize = 110;

// Fused epilogue ("Shared memory and tensor cores", section 13.10: bias,
// activation, residual add or type cast applied to the accumulator before the
// store). kind = 0: plain fp32 store of the accumulator. Otherwise
//   C[m][n] = act(alpha * acc + beta * R[m][n] + bias[n])   (beta = 0: R unread)
// stored as out_dt (DT_F32, DT_F16 or DT_BF16, round to nearest even); R has
// C's element type and may be C itself.
enum Activation { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };
struct Epilogue {
    int kind, act, out_dt, pad;
    float alpha, beta;
    const void* R;
    int64_t ldr;
    const float* bias;
};

// Arguments every kernel receives (by value).
struct GemmArgs {
    const void* A;
    const void* B;
    float* C;
    int64_t lda, ldb, ldc;  // in elements
    int M, N, K;
    int tiles_m, tiles_n;   // ceil(M / bm), ceil(N / bn)
    int group_m;            // tile rows per raster group (L2 locality)
    int xcd_remap;          // 1: give each XCD a contiguous range of tiles
    // Split K (register-staged kernels only): k_split > 1 slices of k_chunk
    // elements; slice blockIdx.y writes its partial product of C to
    // work + y * work_slice with leading dimension work_ld instead of to C.
    int k_split, k_chunk;
    float* work;
    int64_t work_slice, work_ld;
    // Stream-K (persistent software-pipelined kernel only): the last sk_tiles tiles
    // of the linear order are dealt out as equal k-tile shares (streamk.h) to the
    // workgroups blockIdx.x < sk_width; partial sums go to work, slot 2 w + p of
    // 256 x 256 floats. sk_tiles = 0: every tile whole.
    int sk_tiles, sk_width;
    Epilogue ep;            // C's element type is ep.out_dt when ep.kind != 0
};

// One operand copy of a packing launch: rows x cols elements of src (leading
// dimension ld) into a zero-padded rows_p x cols_p destination with leading
// dimension cols_p (a multiple of 16 bytes).
struct PackJob {
    const void* src;
    void* dst;
    int64_t ld;
    int rows, cols;
    int rows_p, cols_p;
};

// Grouped launches ("Grouped Tile Scheduler" of the learn-cutedsl README, section
// 8.4): one persistent grid walks the tiles of several problems. A segment is
// `batch` problems of one shape whose operands sit at fixed element strides
// (batch = 1 for a single problem); its tiles occupy linear tile indices
// [tile_begin, tile_begin + batch * tiles_m * tiles_n). Segments with no tiles are
// left out of the table, so tile_begin is strictly increasing.
struct GroupSeg {
    const void* A;
    const void* B;
    float* C;
    int64_t sa, sb, sc;      // batch strides, in elements
    int64_t tile_begin;
    int lda, ldb, ldc;       // in elements (< 2^23, checked on the host)
    int M, N, K, batch;
    int tiles_m, tiles_n, group_m;
};

// The segment table travels in the kernel arguments (16 x 96 bytes); larger
// groups are split over several launches by the host.
constexpr int kMaxGroupSegments = 16;

struct GroupArgs {
    int count;          // segments in seg[]
    int total_tiles;    // tiles of all segments
    int xcd_remap;      // 1: give each XCD a contiguous block of persistent workgroups
    int pad;
    GroupSeg seg[kMaxGroupSegments];
};

}  // namespace dg
