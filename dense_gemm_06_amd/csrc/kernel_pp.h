// kernel_pp.h -- ping-pong MFMA kernel with direct global -> LDS copies.
#pragma once
#include <type_traits>

#include "lds_layout.h"

namespace dg {

// Ping-pong MFMA kernel for 16-bit inputs on 256 x 256 tiles (K a multiple of 32,
// 16-byte aligned operands; edge tiles in M, and in N for column-major B or for N a
// multiple of 8, copy clamped rows and columns).
//
// The register-staged kernel runs every wave through the same sequence (load,
// wait, MFMA, store, barrier), so the matrix unit idles whenever all waves wait
// on memory together. Here the 8 waves form two groups of 4, one wave of each
// group per SIMD, and the groups run one phase apart: in every phase one group
// issues a block of MFMAs from registers while the other reads its fragments of
// the next k-tile from LDS and starts direct global -> LDS copies
// (global_load_lds_dwordx4, no registers involved) three k-tiles ahead. One
// barrier ends each phase. MF selects the matrix instruction: 16 for
// v_mfma_f32_16x16x32 (32 per phase), 32 for v_mfma_f32_32x32x16 (16 per phase).
//
// LDS: 4 stages of 32 KB (A: 256 rows x 32 k, B: 32 k x 256 n or 256 n x 32 k).
// Group 0 computes C rows 0..127 of the tile and copies A; group 1 computes rows
// 128..255 and copies B; wave w of a group owns columns 64w..64w+63.
// Tile q lives in stage q mod 4: group 0 reads it in phase 2q, group 1 in phase
// 2q+1, and its stage is refilled (tile q+4) from phase 2q+2 on. Before each
// barrier a wave waits for its own LDS reads (so a stage is never overwritten
// while read) and, before the barrier that precedes phase 2q, for its own copies
// of tile q (vmcnt counts its copies of tiles q+1 and q+2 still in flight).
//
// The chunk swizzles follow the fragment shape: kmaj64_swz / nmaj_swz for 16-row
// fragments, kmaj32_swz / nmaj32_swz for 32-row fragments.
template <int DT, int OPB, int MF>
__global__ __launch_bounds__(512) void mfma16_pp(GemmArgs g) {
    static_assert(MF == 16 || MF == 32, "MFMA shape");
    constexpr int BM = 256, BN = 256, BK = 32, S = 4;
    constexpr int SA = BM * BK, SB = BN * BK;  // halfs per stage
    __shared__ __attribute__((aligned(1024))) uint16_t sA[S][SA];
    __shared__ __attribute__((aligned(1024))) uint16_t sB[S][SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, wl = wave & 3;
    const int l16 = lane & 15, lg = lane >> 4;
    const int l32 = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = g.K / BK;
    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.B);
    // chunk swizzles of the k-major tiles (64-byte rows) and of the row-major B tile,
    // chosen per fragment shape (16 or 32 rows per read)
    auto kswz = [](int r) { return MF == 16 ? kmaj64_swz(r) : kmaj32_swz(r); };
    auto nswz = [](int k) { return MF == 16 ? nmaj_swz<BN / 8>(k) : nmaj32_swz(k); };

    // Direct copies: each wave issues 4 copies of 1 KB (64 lanes x 16 B) per tile.
    // Lane L of block b lands at LDS byte b*1024 + 16L, i.e. at a fixed swizzled
    // position; it loads the logical chunk that belongs there. Edge tiles (M or N not
    // a multiple of 256): rows at or beyond M (N) copy row M - 1 (N - 1), and column
    // chunks of a row-major B at or beyond N copy columns 0..7 (N is then a multiple
    // of 8); the masked epilogue never stores what they produce.
    const uint16_t* src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = wl * 4 + i;
        if (grp == 0 || OPB == 1) {
            const int row = b * 16 + (lane >> 2);
            const int c = (lane & 3) ^ kswz(row);
            src[i] = grp == 0 ? A + (size_t)min(m0 + row, g.M - 1) * g.lda + c * 8
                              : B + (size_t)min(n0 + row, g.N - 1) * g.ldb + c * 8;
        } else {
            const int row = b * 2 + (lane >> 5);
            const int c = (lane & 31) ^ nswz(row);
            const int col = n0 + c * 8;
            src[i] = B + (size_t)row * g.ldb + (col < g.N ? col : 0);
        }
    }
    const size_t kstep = (grp == 1 && OPB == 0) ? (size_t)BK * g.ldb : (size_t)BK;  // elements per k-tile
    auto issue = [&](int t) {
        uint16_t* dst = grp == 0 ? sA[t & 3] : sB[t & 3];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(DG_GLB(src[i] + (size_t)t * kstep), DG_LDSV(dst + (wl * 4 + i) * 512), 16,
                                             0, 0);
    };

    // Fragments of one k-tile, in NF k steps (one per MFMA depth): qa = Q fragments
    // (A rows), pb = P fragments of column-major B, ph = the two 4-k halves of a
    // row-major-B P fragment, read by transpose reads issued as inline asm. The
    // compiler cannot tell those reads from the in-flight LDS-DMA writes and would
    // otherwise wait for every copy (vmcnt(0)) before them; the asm form leaves the
    // ordering to the explicit waits of sync_phase. Their results are combined into
    // MFMA operands only after the lgkmcnt(0) wait and barrier that end the phase.
    //   MF = 16: v_mfma_f32_16x16x32, wave tile 128 x 64 = 8 x 4 subtiles, one k step;
    //            lane supplies row/column l16, k 8*lg .. 8*lg+7
    //   MF = 32: v_mfma_f32_32x32x16, wave tile 128 x 64 = 4 x 2 subtiles, two k steps
    //            of 16; lane supplies row/column l32, k 16*ks + 8*lh .. +7
    constexpr int NF = MF == 16 ? 1 : 2;        // k steps per tile
    constexpr int SI = MF == 16 ? 8 : 4;        // subtile rows per wave
    constexpr int SJ = MF == 16 ? 4 : 2;        // subtile columns per wave
    u32x4 qa[NF][SI], pb[NF][SJ];
    u32x2 ph[NF][SJ][2];
    auto load_frags = [&](int t) {
        const uint16_t* a = sA[t & 3];
        const uint16_t* bb = sB[t & 3];
#pragma unroll
        for (int ks = 0; ks < NF; ++ks) {
#pragma unroll
            for (int i = 0; i < SI; ++i) {
                const int r = grp * 128 + i * MF + (MF == 16 ? l16 : l32);
                const int c = MF == 16 ? lg : ks * 2 + lh;
                qa[ks][i] = *reinterpret_cast<const u32x4*>(a + r * BK + ((c ^ kswz(r)) << 3));
            }
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                if (OPB == 0) {
                    // transpose reads: in each 16-lane group, lane i addresses row kb + i/4 at
                    // columns nb + 4(i%4); lane i then holds column nb + i of rows kb..kb+3.
                    // MF = 32: lane groups 0/1 (2/3) cover columns 0-15 / 16-31 of k rows
                    // 0-7 (8-15) of the step.
                    const int col = MF == 16 ? wl * 64 + j * 16 + ((l16 & 3) << 2)
                                             : wl * 64 + j * 32 + (lg & 1) * 16 + ((l16 & 3) << 2);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int krow = MF == 16 ? lg * 8 + hh * 4 + (l16 >> 2)
                                                  : ks * 16 + (lg >> 1) * 8 + hh * 4 + (l16 >> 2);
                        const uint16_t* p = bb + krow * BN + (((col >> 3) ^ nswz(krow)) << 3) + (col & 7);
                        const uint32_t addr = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(p));
                        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(ph[ks][j][hh]) : "v"(addr));
                    }
                } else {
                    const int r = wl * 64 + j * MF + (MF == 16 ? l16 : l32);
                    const int c = MF == 16 ? lg : ks * 2 + lh;
                    pb[ks][j] = *reinterpret_cast<const u32x4*>(bb + r * BK + ((c ^ kswz(r)) << 3));
                }
            }
        }
    };

    using AccT = typename std::conditional<MF == 16, f32x4, f32x16>::type;
    AccT acc[SI][SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j) acc[i][j] = AccT{};
    auto mma = [&]() {
        if (OPB == 0) {
#pragma unroll
            for (int ks = 0; ks < NF; ++ks)
#pragma unroll
                for (int j = 0; j < SJ; ++j)
                    pb[ks][j] = u32x4{ph[ks][j][0][0], ph[ks][j][0][1], ph[ks][j][1][0], ph[ks][j][1][1]};
        }
#pragma unroll
        for (int ks = 0; ks < NF; ++ks)
#pragma unroll
            for (int i = 0; i < SI; ++i)
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    if constexpr (MF == 16) {
                        if (DT == DT_F16)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8, pb[ks][j]), __builtin_bit_cast(f16x8, qa[ks][i]), acc[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, pb[ks][j]), __builtin_bit_cast(bf16x8, qa[ks][i]), acc[i][j], 0, 0, 0);
                    } else {
                        if (DT == DT_F16)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                __builtin_bit_cast(f16x8, pb[ks][j]), __builtin_bit_cast(f16x8, qa[ks][i]), acc[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, pb[ks][j]), __builtin_bit_cast(bf16x8, qa[ks][i]), acc[i][j], 0, 0, 0);
                    }
                }
    };
    // End of a phase: own LDS reads done, then (optionally) own copies of the next
    // tile done, then the workgroup barrier. The asm statements are compiler
    // memory barriers; the waits are explicit because LDS-DMA completion is not
    // tracked by the compiler for later LDS reads.
    auto sync_phase = [&](int vm_allowed) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (vm_allowed >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (vm_allowed >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else if (vm_allowed >= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
    };

    // prologue: tiles 0, 1, 2 in flight; tile 0 complete before the first phase
    for (int t = 0; t < 3 && t < nk; ++t) issue(t);
    sync_phase(4 * min(2, nk - 1));

    for (int q = 0; q < nk; ++q) {
        // phase 2q: group 0 fetches tile q, group 1 multiplies tile q-1
        if (grp == 0) {
            load_frags(q);
            if (q + 3 < nk) issue(q + 3);
        } else if (q > 0) {
            mma();
        }
        sync_phase(-1);
        // phase 2q+1: group 0 multiplies tile q, group 1 fetches tile q
        if (grp == 0) {
            mma();
        } else {
            load_frags(q);
            if (q + 3 < nk) issue(q + 3);
        }
        sync_phase(4 * max(0, min(2, nk - 2 - q)));
    }
    if (grp == 1) mma();

    if constexpr (MF == 16) {
        if (g.ep.kind != 0) {
            // Fused epilogue, staged through LDS (free once every wave's last fragment
            // reads are done): each wave writes half of its 128 x 64 fp32 tile into its
            // own 16 KB slot (chunk c of row r at c ^ (r & 15): conflict-free writes of the
            // fragment layout and reads of whole rows), then reads back whole rows,
            // 4 columns per lane, and applies the epilogue with coalesced row stores.
            // Only this wave touches its slot; the wave barrier keeps the compiler from
            // moving LDS accesses across the write/read phases, which the hardware
            // executes in order within a wave.
            __syncthreads();
            char* slot = reinterpret_cast<char*>(grp == 0 ? &sA[0][0] : &sB[0][0]) + wl * 16384;
            const int cm0 = m0 + grp * 128, cn0 = n0 + wl * 64;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int row = ii * 16 + l16;
#pragma unroll
                    for (int j = 0; j < SJ; ++j) {
                        const int chunk = j * 4 + lg;
                        *reinterpret_cast<f32x4*>(slot + row * 256 + ((chunk ^ (row & 15)) << 4)) = acc[h * 4 + ii][j];
                    }
                }
                __builtin_amdgcn_wave_barrier();
                for (int it = 0; it < 16; ++it) {
                    const int row = it * 4 + (lane >> 4), chunk = lane & 15;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(slot + row * 256 + ((chunk ^ (row & 15)) << 4));
                    const int m = cm0 + h * 64 + row;
                    if (m < g.M) epilogue_run4_body(g.ep, g.C, g.ldc, g.N, m, cn0 + chunk * 4, v);
                }
                __builtin_amdgcn_wave_barrier();
            }
            return;
        }
    }

    // epilogue: lane owns C[m][n..n+3]; 16x16: one run per subtile (n = 4*lg ..);
    // 32x32: register r of the subtile holds row n = 8(r/4) + 4*lh + r%4, so four runs.
    // The operands may be zero-padded copies larger than C (whole tiles): rows >= M
    // and columns >= N of the padded product are not stored.
#pragma unroll
    for (int i = 0; i < SI; ++i) {
        const int m = m0 + grp * 128 + i * MF + (MF == 16 ? l16 : l32);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < SJ; ++j)
#pragma unroll
            for (int rg = 0; rg < (MF == 16 ? 1 : 4); ++rg) {
                const int n = n0 + wl * 64 + j * MF + (MF == 16 ? lg * 4 : rg * 8 + lh * 4);
                // plain stores (the 16x16 form runs its epilogue staged above; the 32x32
                // form is plain-store only)
                store_run4<false>(g, m, n, f32x4{acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2],
                                                 acc[i][j][4 * rg + 3]});
            }
    }
}

}  // namespace dg
