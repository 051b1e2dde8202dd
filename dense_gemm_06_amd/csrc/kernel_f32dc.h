// kernel_f32dc.h -- fp32 64 x 64 tiles with direct global -> LDS copies several
// k-tiles ahead (schedule 8).
#pragma once
#include "kernel_sp.h"

namespace dg {

// fp32 inputs on v_mfma_f32_16x16x4_f32, one 64 x 64 tile of C per workgroup, K split
// over KG groups of four waves (group kg takes k-tiles kg, kg + KG, ...; K is a
// multiple of KG * 32, checked by the host). Each wave owns a 16 x 64 slice of the
// tile, as in the register-staged 64 x 64 tile (fragments, MFMA order and store are
// that kernel's), but the operands reach LDS by direct copies (global_load_lds, 16
// bytes per lane: one instruction fills 1 KB of LDS) into S stages per group, issued
// S - 1 k-tiles ahead. Nothing passes through registers, so a copy can be in flight
// for S - 2 whole k-tiles before its data is needed, and the k loop carries no
// address or store arithmetic for the staging.
//
// Iteration lt (stage lt % S): copy k-tile lt + S - 1 into the stage of k-tile lt - 1
// (whose reads ended before the previous barrier); read the second half of k-tile
// lt's fragments; MFMAs on the first half; read the first half of k-tile lt + 1
// (complete and published by the previous barrier); MFMAs on the second half; wait
// until this wave's copies of k-tile lt + 2 have landed; barrier. Only copies are in
// flight in the loop (no stores), so the vector-memory counter counts copies alone
// and they complete in order.
//
// LDS layouts (those of the register-staged fp32 tile): A, and B when column-major,
// k-major rows of 32 floats, chunk c of row r at position c ^ (r & 7); a row-major B
// as k-rows of 64 floats, unswizzled. Copy block b of A fills rows 8b .. 8b + 7: lane
// L lands at byte 16 L of the block, position L & 7 of row 8b + (L >> 3), and loads
// the logical chunk that belongs there. Edge tiles: rows of A (and of a
// column-major B) at or beyond M (N) copy row M - 1 (N - 1); 16-byte column chunks of
// a row-major B at or beyond N (a multiple of 4) copy columns 0 .. 3. What they bring
// in reaches only rows and columns of C that are not stored.
template <int OPB, int KG, int S>
__global__ __launch_bounds__(256 * KG) void mfma32_dc(GemmArgs g) {
    k_slice<4, OPB>(g);  // a split-K launch: this workgroup's slice (whole pairs of k-tiles)
    constexpr int BM = 64, BN = 64, BK = 32;
    constexpr int NT = 256;                  // threads per K group
    constexpr int STAGE = BM * BK;           // floats per operand and stage (B: BK x BN, the same)
    constexpr int STAGE_BYTES = STAGE * 4;   // 8 KB
    static_assert(KG == 1 || KG == 2, "k groups");
    static_assert(S >= 3 && KG * S * 2 * STAGE_BYTES <= 160 * 1024, "stages");
    __shared__ __attribute__((aligned(1024))) float sAg[KG][S][STAGE];
    __shared__ __attribute__((aligned(1024))) float sBg[KG][S][STAGE];

    const int kg = KG == 1 ? 0 : (int)threadIdx.x / NT;  // uniform per wave
    const int tid = (int)threadIdx.x - kg * NT, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const float* __restrict__ A = static_cast<const float*>(g.A);
    const float* __restrict__ B = static_cast<const float*>(g.B);
    const int nl = g.K / (BK * KG);  // k-tiles per group

    // Copy sources at this group's first k-tile, and the step between its k-tiles.
    // Wave w copies blocks 2w and 2w + 1 of A and of B.
    const float* srcA[2];
    const float* srcB[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int b = 2 * wave + i;
        const int row = b * 8 + (lane >> 3), c = (lane & 7) ^ kmaj_swz(row);
        srcA[i] = A + (size_t)min(m0 + row, g.M - 1) * g.lda + kg * BK + 4 * c;
        if (OPB == 1) {
            srcB[i] = B + (size_t)min(n0 + row, g.N - 1) * g.ldb + kg * BK + 4 * c;
        } else {
            const int krow = b * 4 + (lane >> 4), col = n0 + 4 * (lane & 15);
            srcB[i] = B + (size_t)(kg * BK + krow) * g.ldb + (col < g.N ? col : 0);
        }
    }
    const size_t stepA = (size_t)KG * BK;
    const size_t stepB = OPB == 0 ? (size_t)KG * BK * g.ldb : (size_t)KG * BK;
    const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t dstA = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sAg[kg][0][0])) + wave_u * 2048u;
    const uint32_t dstB = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sBg[kg][0][0])) + wave_u * 2048u;
    auto issue = [&](int lt, uint32_t st) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(DG_GLB(srcA[i] + (size_t)lt * stepA),
                                             DG_LDS_AT(dstA + st * STAGE_BYTES + i * 1024u), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(DG_GLB(srcB[i] + (size_t)lt * stepB),
                                             DG_LDS_AT(dstB + st * STAGE_BYTES + i * 1024u), 16, 0, 0);
    };

    // Fragments of one half k-tile (16 k): A rows wave*16 + l16 as a float4 along k;
    // B as four k-rows (row-major: a float4 along n) or four 16-column subtiles
    // (column-major: a float4 along k).
    struct Frag {
        f32x4 a;
        f32x4 b[4];
    };
    const int ra = wave * 16 + l16;
    auto read_frag = [&](Frag& f, uint32_t st, int kk) {
        const float* sa = &sAg[kg][0][0] + st * STAGE;
        const float* sb = &sBg[kg][0][0] + st * STAGE;
        f.a = *reinterpret_cast<const f32x4*>(sa + ra * BK + ((((kk >> 2) + lg) ^ kmaj_swz(ra)) << 2));
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (OPB == 0) {
                f.b[s] = *reinterpret_cast<const f32x4*>(sb + (kk + 4 * lg + s) * BN + 4 * l16);
            } else {
                const int r = s * 16 + l16;
                f.b[s] = *reinterpret_cast<const f32x4*>(sb + r * BK + ((((kk >> 2) + lg) ^ kmaj_swz(r)) << 2));
            }
        }
    };
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto read_one = [&](Frag& f, uint32_t st, int kk, int r) {
        const float* sa = &sAg[kg][0][0] + st * STAGE;
        const float* sb = &sBg[kg][0][0] + st * STAGE;
        if (r == 0) {
            f.a = *reinterpret_cast<const f32x4*>(sa + ra * BK + ((((kk >> 2) + lg) ^ kmaj_swz(ra)) << 2));
        } else if (OPB == 0) {
            f.b[r - 1] = *reinterpret_cast<const f32x4*>(sb + (kk + 4 * lg + r - 1) * BN + 4 * l16);
        } else {
            const int rb = (r - 1) * 16 + l16;
            f.b[r - 1] = *reinterpret_cast<const f32x4*>(sb + rb * BK + ((((kk >> 2) + lg) ^ kmaj_swz(rb)) << 2));
        }
    };
    // The 16 MFMAs of one half, with the five fragment reads of another half after the
    // MFMAs at positions rpos .. rpos + 4 and, with a copy tag, this wave's four copies
    // of k-tile ct into stage cst after MFMAs 1, 3, 5 and 7, so that the matrix unit
    // starts right after the barrier and the other instructions issue in its shadow.
    auto mma_mixed = [&](const Frag& f, Frag& nf, uint32_t nst, int nkk, int rpos, bool copy, int ct, uint32_t cst) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = 4 * s + j;
                if (OPB == 0)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[s][j], f.a[s], acc[j], 0, 0, 0);
                else
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[j][s], f.a[s], acc[j], 0, 0, 0);
                if (k >= rpos && k < rpos + 5) read_one(nf, nst, nkk, k - rpos);
                if (copy && (k & 1) && k < 8) {
                    const int i = (k >> 1) & 1;
                    if (k < 4)
                        __builtin_amdgcn_global_load_lds(DG_GLB(srcA[i] + (size_t)ct * stepA),
                                                         DG_LDS_AT(dstA + cst * STAGE_BYTES + i * 1024u), 16, 0, 0);
                    else
                        __builtin_amdgcn_global_load_lds(DG_GLB(srcB[i] + (size_t)ct * stepB),
                                                         DG_LDS_AT(dstB + cst * STAGE_BYTES + i * 1024u), 16, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    };
    auto settle = [&](Frag& f) {
        asm volatile("" : "+v"(f.a), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
    };

    // prologue: k-tiles 0 .. S - 2 in flight; k-tiles 0 and 1 complete
    for (int t = 0; t < S - 1 && t < nl; ++t) issue(t, (uint32_t)t);
    vm_wait(4 * max(0, min(S - 2, nl - 1) - 1));
    asm volatile("s_barrier" ::: "memory");
    Frag f0, f1;
    if (nl > 0) read_frag(f0, 0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(f0);
    uint32_t st = 0;  // lt % S
    // One iteration; COPY: k-tile lt + S - 1 exists and is copied, and then the wait
    // leaves the copies of k-tiles lt + 3 .. lt + S - 1 in flight.
    auto iteration = [&](int lt, auto copy_tag) {
        constexpr bool COPY = decltype(copy_tag)::value;
        const uint32_t nst = st + 1 == S ? 0 : st + 1;
        const uint32_t cst = st == 0 ? S - 1 : st - 1;  // (lt + S - 1) % S
        // first half: the second half's fragments read after its first MFMAs
        mma_mixed(f0, f1, st, 16, 0, false, 0, 0);
        // second half: the copies of k-tile lt + S - 1 (into the stage of k-tile lt - 1)
        // and the first half of k-tile lt + 1 (unconditional: after the last k-tile it
        // reads a stage whose values go unused)
        mma_mixed(f1, f0, nst, 0, 8, COPY, lt + S - 1, cst);
        // this wave's copies of k-tile lt + 2 landed (those of later k-tiles may be in
        // flight), its own LDS reads done; then the barrier publishes k-tile lt + 2 and
        // frees stage st for the copies of the next iteration
        if (COPY) vm_wait_n<4 * (S - 3)>();
        else vm_wait(4 * max(0, nl - 1 - (lt + 2)));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        settle(f0);
        st = nst;
    };
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    int lt = 0;
    for (; lt + S - 1 < nl; ++lt) iteration(lt, yes);
    for (; lt < nl; ++lt) iteration(lt, no);

    if constexpr (KG == 2) {
        // group 1's accumulators through LDS (its own A stages: every copy has landed
        // and every read of them is done), lane-major; group 0 adds them after its own
        // (a fixed order)
        static_assert(4 * 4 * 64 * 4 <= S * STAGE, "reduction buffer");
        float* red = &sAg[1][0][0];
        if (kg == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[((wave * 4 + j) * 4 + e) * 64 + lane] = acc[j][e];
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] += red[((wave * 4 + j) * 4 + e) * 64 + lane];
    }

    const int m = m0 + ra;
    if (m >= g.M) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (OPB == 0) {
            // subtile j holds columns 4 l16 + j: lane owns 16 consecutive n of row m
            const int n = n0 + 16 * lg + 4 * r;
            store_run4(g, m, n, f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]});
        } else {
            const int n = n0 + r * 16 + lg * 4;
            store_run4(g, m, n, acc[r]);
        }
    }
}

}  // namespace dg

namespace dg {

// fp32 inputs on v_mfma_f32_16x16x4_f32, BM x BN tiles (256 x 128 or 128 x 128) on
// eight waves (schedule 9): a WM x WN grid of wave tiles of (BM / WM) x 64, operands
// copied straight into S LDS stages of k = 32 (global_load_lds, 16 bytes per lane,
// 1 KB per instruction). Each wave holds FA = BM / WM / 16 row blocks of A and, per
// k-step, 64 columns of B as four strided 16-column blocks (row-major B: column
// 4 l16 + j of the wave tile in block j, one float4 read along n per k-row;
// column-major B: four contiguous 16-column blocks, a float4 along k each).
//
// Iteration lt (stage lt % S): the copies of k-tile lt + S - 1 (into the stage of
// k-tile lt - 1, whose reads ended before the previous barrier) and the reads of
// k-tile lt's second half go out between the first half's MFMAs; the second half's
// MFMAs carry the reads of k-tile lt + 1's first half (published by the previous
// barrier); then this wave's copies of k-tile lt + 2 must have landed, and a barrier
// publishes it. With three stages (256 x 128) the copies of k-tile lt + 2 are waited
// for at the end of the iteration that issues them, a whole iteration (128 MFMAs per
// wave) after they went out; with five (128 x 128), two iterations later.
//
// LDS layouts: A (and a column-major B) as in the 64 x 64 direct-copy tile, k-major
// rows of 32 floats, chunk c of row r at c ^ (r & 7). A row-major B in 64-column
// segments of 8 KB (one per wave-tile column), each made of 1 KB blocks of four
// k-rows: block a holds k-rows 4a .. 4a + 3, its 256-byte window q their 64-byte
// quads q (columns 16 q .. 16 q + 15), k-row 4a + t at slot t ^ q. Every 16-lane phase
// of a fragment read (four k-rows, 16 columns each) is then free of bank conflicts and
// puts four lanes in each 256-byte window of the 1 KB period; with the plain k-row
// layout of the 64 x 64 tile (all four k-rows in one window) the same reads ran 17-25%
// slower here. (That tile, with its one-row-block wave tiles, measured 0-5% slower
// with this layout and keeps its own.) Edge tiles: rows past M (N) copy row M - 1
// (N - 1); 16-byte column chunks of a row-major B at or past N (a multiple of 4) copy
// columns 0 .. 3; neither reaches a stored element.
template <int OPB, int BM, int BN, int S>
__global__ __launch_bounds__(512) void mfma32_dcl(GemmArgs g) {
    k_slice<4, OPB>(g);  // a split-K launch: this workgroup's slice (whole k-tiles)
    constexpr int BK = 32, NW = 8;
    constexpr int WN = BN / 64, WM = NW / WN, WTM = BM / WM, FA = WTM / 16;
    static_assert(BN % 64 == 0 && NW % WN == 0 && WTM % 16 == 0 && FA >= 1 && FA <= 4, "wave grid");
    constexpr int SA = BM * BK, SB = BK * BN;  // floats per stage
    constexpr int CA = BM / 64, CB = BN / 64;  // 1 KB copies per wave and k-tile
    constexpr int CPW = CA + CB;
    constexpr int NR = FA + 4;                 // fragment reads per half k-tile
    static_assert(S >= 3 && S * (SA + SB) * 4 <= 160 * 1024, "stages");
    static_assert(2 * CPW <= 16 * FA && NR + 8 <= 16 * FA, "interleave slots");
    __shared__ __attribute__((aligned(1024))) float sA[S * SA];
    __shared__ __attribute__((aligned(1024))) float sB[S * SB];

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const float* __restrict__ A = static_cast<const float*>(g.A);
    const float* __restrict__ B = static_cast<const float*>(g.B);
    const int nl = g.K / BK;

    // Copy sources at k-tile 0: wave w copies blocks w CA .. w CA + CA - 1 of A (8 rows
    // each) and w CB .. w CB + CB - 1 of B.
    const float* srcA[CA];
    const float* srcB[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int row = (wave * CA + i) * 8 + (lane >> 3), c = (lane & 7) ^ kmaj_swz(row);
        srcA[i] = A + (size_t)min(m0 + row, g.M - 1) * g.lda + 4 * c;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int b = wave * CB + i;
        if (OPB == 1) {
            const int row = b * 8 + (lane >> 3), c = (lane & 7) ^ kmaj_swz(row);
            srcB[i] = B + (size_t)min(n0 + row, g.N - 1) * g.ldb + 4 * c;
        } else {
            // block b: k-rows 4a .. 4a + 3 (a = b % 8) of the 64-column segment b / 8; its
            // 256-byte window q holds their 64-byte quads q (columns 16 q .. 16 q + 15),
            // k-row 4a + t at slot t ^ q. Lane L fills window L / 16, slot (L / 4) % 4,
            // chunk L % 4.
            const int seg = b >> 3, a = b & 7, q = lane >> 4, t = (lane >> 2) & 3, e = lane & 3;
            const int krow = 4 * a + (t ^ q), col = n0 + seg * 64 + 16 * q + 4 * e;
            srcB[i] = B + (size_t)krow * g.ldb + (col < g.N ? col : 0);
        }
    }
    const size_t stepB = OPB == 0 ? (size_t)BK * g.ldb : (size_t)BK;
    const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t dstA = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sA[0])) + wave_u * (CA * 1024u);
    const uint32_t dstB = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sB[0])) + wave_u * (CB * 1024u);
    // copy q (0 .. CPW - 1) of this wave's share of k-tile lt into stage st
    auto copy_one = [&](int q, int lt, uint32_t st) {
        if (q < CA)
            __builtin_amdgcn_global_load_lds(DG_GLB(srcA[q] + (size_t)lt * BK),
                                             DG_LDS_AT(dstA + st * (SA * 4u) + q * 1024u), 16, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(DG_GLB(srcB[q - CA] + (size_t)lt * stepB),
                                             DG_LDS_AT(dstB + st * (SB * 4u) + (q - CA) * 1024u), 16, 0, 0);
    };

    struct Frag {
        f32x4 a[FA];
        f32x4 b[4];
    };
    const int ra0 = wm * WTM + l16;
    // read r (0 .. NR - 1) of the fragments of the half k-tile at kk of stage st
    auto read_one = [&](Frag& f, uint32_t st, int kk, int r) {
        const float* sa = sA + st * SA;
        const float* sb = sB + st * SB;
        if (r < FA) {
            const int ra = ra0 + 16 * r;
            f.a[r] = *reinterpret_cast<const f32x4*>(sa + ra * BK + ((((kk >> 2) + lg) ^ kmaj_swz(ra)) << 2));
        } else if (OPB == 0) {
            const int kr = kk + 4 * lg + r - FA, q = l16 >> 2;
            f.b[r - FA] = *reinterpret_cast<const f32x4*>(sb + wn * (BK * 64) + (kr >> 2) * 256 + q * 64 +
                                                          (((kr & 3) ^ q) << 4) + 4 * (l16 & 3));
        } else {
            const int rb = wn * 64 + (r - FA) * 16 + l16;
            f.b[r - FA] = *reinterpret_cast<const f32x4*>(sb + rb * BK + ((((kk >> 2) + lg) ^ kmaj_swz(rb)) << 2));
        }
    };
    f32x4 acc[FA][4];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The 16 FA MFMAs of one half, with the NR reads of another half after the MFMAs
    // at positions rpos .. rpos + NR - 1 and, with a copy tag, this wave's CPW copies
    // of k-tile ct into stage cst after MFMAs 1, 3, 5, ...
    auto mma_mixed = [&](const Frag& f, Frag& nf, uint32_t nst, int nkk, int rpos, bool copy, int ct, uint32_t cst) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < FA; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = (s * FA + i) * 4 + j;
                    if (OPB == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[s][j], f.a[i][s], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[j][s], f.a[i][s], acc[i][j], 0, 0, 0);
                    if (k >= rpos && k < rpos + NR) read_one(nf, nst, nkk, k - rpos);
                    if (copy && (k & 1) && (k >> 1) < CPW) copy_one(k >> 1, ct, cst);
                    __builtin_amdgcn_sched_barrier(0);
                }
    };
    auto settle = [&](Frag& f) {
#pragma unroll
        for (int i = 0; i < FA; ++i) asm volatile("" : "+v"(f.a[i]));
#pragma unroll
        for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(f.b[s]));
    };

    // prologue: k-tiles 0 .. S - 2 in flight; k-tiles 0 and 1 complete
    for (int t = 0; t < S - 1 && t < nl; ++t)
#pragma unroll
        for (int q = 0; q < CPW; ++q) copy_one(q, t, (uint32_t)t);
    vm_wait(CPW * max(0, min(S - 2, nl - 1) - 1));
    asm volatile("s_barrier" ::: "memory");
    Frag f0, f1;
    if (nl > 0)
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(f0, 0, 0, r);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(f0);
    uint32_t st = 0;  // lt % S
    // One iteration; COPY: k-tile lt + S - 1 exists and is copied, and the wait then
    // leaves the copies of k-tiles lt + 3 .. lt + S - 1 in flight.
    auto iteration = [&](int lt, auto copy_tag) {
        constexpr bool COPY = decltype(copy_tag)::value;
        const uint32_t nst = st + 1 == S ? 0 : st + 1;
        const uint32_t cst = st == 0 ? S - 1 : st - 1;  // (lt + S - 1) % S
        // first half: the copies of k-tile lt + S - 1 and the second half's fragments
        mma_mixed(f0, f1, st, 16, 0, COPY, lt + S - 1, cst);
        // second half: the first half of k-tile lt + 1 (unconditional: after the last
        // k-tile it reads a stage whose values go unused)
        mma_mixed(f1, f0, nst, 0, 8, false, 0, 0);
        if (COPY) vm_wait_n<CPW * (S - 3)>();
        else vm_wait(CPW * max(0, nl - 1 - (lt + 2)));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        settle(f0);
        st = nst;
    };
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    int lt = 0;
    for (; lt + S - 1 < nl; ++lt) iteration(lt, yes);
    for (; lt < nl; ++lt) iteration(lt, no);

#pragma unroll
    for (int i = 0; i < FA; ++i) {
        const int m = m0 + ra0 + 16 * i;
        if (m >= g.M) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (OPB == 0) {
                // block j holds wave-tile columns 4 l16 + j: the lane owns 16 consecutive n
                const int n = n0 + wn * 64 + 16 * lg + 4 * r;
                store_run4(g, m, n, f32x4{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]});
            } else {
                const int n = n0 + wn * 64 + r * 16 + lg * 4;
                store_run4(g, m, n, acc[i][r]);
            }
        }
    }
}

}  // namespace dg
