// kernel_w4.h -- four-wave software-pipelined MFMA kernel (one wave per SIMD).
#pragma once
#include <type_traits>

#include "lds_layout.h"

// An LDS pointer made from a byte address (an integer): it carries no link to the
// LDS variable the address falls in.
#define DG_LDS_AT(a) ((__attribute__((address_space(3))) void*)(uintptr_t)(uint32_t)(a))

namespace dg {

// Software-pipelined MFMA kernel for 16-bit inputs on full 256 x 256 tiles (M and
// N multiples of 256, K a multiple of 32, 16-byte aligned operands).
//
// Four waves, one per SIMD, each own a 128 x 128 quarter of the tile (2 x 2 wave
// grid) and keep its 16 v_mfma_f32_32x32x16 accumulators (256 registers) in the
// accumulation registers. A wave of 128 x 128 reads 64 bytes of LDS fragments per
// 32x32x16 MFMA, against 96 for the 128 x 64 waves of the eight-wave layouts, and a
// single wave keeps this instruction's issue rate near peak, which two waves per
// SIMD would otherwise be needed for with 16x16x32.
//
// The k loop runs in steps of 16. Each wave holds two fragment sets: while the 16
// MFMAs of step s run from one set, the fragment reads of step s+1 fill the other,
// interleaved with the MFMAs. Tiles of k = 32 (two steps) arrive by direct
// global -> LDS copies (global_load_lds_dwordx4) into a ring of S stages, issued
// S-1 tiles ahead: a wave copies 4 KB of A during the first step of a tile and 4
// KB of B during the second. One barrier per tile, between its two steps, makes
// the next tile visible (each wave first waits for its own copies of it) and
// retires the stage the refill of the current iteration overwrites.
//
// Tile t sits in stage t mod S. Step (t, 0)'s fragments are read during step
// (t-1, 1), step (t, 1)'s during step (t, 0). The last reads of stage t mod S are
// therefore done (lgkmcnt(0)) before the barrier of iteration t, and iteration
// t+1 refills that stage with tile t+S.
//
// LDS layouts and the fragment maps are those of the 32x32x16 ping-pong form:
// k-major 64-byte rows with chunk swizzle kmaj32_swz, row-major B with nmaj32_swz,
// read through ds_read_b64_tr_b16. Both swizzles depend on the lane only for the
// rows a wave reads, so every fragment read is a per-lane base plus an immediate.
// Wait until at most n (a multiple of 4, below 32) of this wave's vector memory
// operations are in flight.
template <int N>
__device__ __forceinline__ void vm_wait_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void vm_wait(int n) {
    switch (n) {
        case 0: vm_wait_n<0>(); break;
        case 4: vm_wait_n<4>(); break;
        case 8: vm_wait_n<8>(); break;
        case 12: vm_wait_n<12>(); break;
        case 16: vm_wait_n<16>(); break;
        case 20: vm_wait_n<20>(); break;
        case 24: vm_wait_n<24>(); break;
        default: vm_wait_n<0>(); break;
    }
}

template <int DT, int OPB, int S = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma32_w4(GemmArgs g) {
    static_assert(S >= 3 && S <= 5, "stages");
    constexpr int BM = 256, BN = 256, BK = 32, D = S - 1;  // D: copy distance in tiles
    constexpr int SA = BM * BK, SB = BN * BK;      // halfs per stage
    constexpr int STAGE_BYTES = SA * 2;            // 16 KB for each of A and B
    __shared__ __attribute__((aligned(1024))) uint16_t sA[S][SA];  // S = 5: all 160 KB
    __shared__ __attribute__((aligned(1024))) uint16_t sB[S][SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int l16 = lane & 15, lg = lane >> 4;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = g.K / BK;
    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.B);

    // ---- direct copies: wave w moves blocks 4w..4w+3 (1 KB each) of the A tile and
    // of the B tile. Lane L of block b lands at LDS byte b*1024 + 16L, a fixed
    // swizzled position, and loads the logical 16-byte chunk that belongs there.
    const uint16_t* srcA[4];
    const uint16_t* srcB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = wave * 4 + i;
        const int row = b * 16 + (lane >> 2);
        srcA[i] = A + (size_t)(m0 + row) * g.lda + (((lane & 3) ^ kmaj32_swz(row)) << 3);
        if (OPB == 1) {
            srcB[i] = B + (size_t)(n0 + row) * g.ldb + (((lane & 3) ^ kmaj32_swz(row)) << 3);
        } else {
            const int krow = b * 2 + (lane >> 5);
            srcB[i] = B + (size_t)krow * g.ldb + n0 + (((lane & 31) ^ nmaj32_swz(krow)) << 3);
        }
    }
    const size_t kstepB = OPB == 0 ? (size_t)BK * g.ldb : (size_t)BK;  // elements per k-tile
    // LDS destinations as plain wave-uniform numbers (M0 takes them directly). Built
    // from an integer, a copy's LDS pointer carries no link to sA / sB, so the
    // compiler does not make every later LDS read wait for all copies in flight
    // (vmcnt(0)); the explicit waits below order them instead.
    const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t dstA = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sA[0][0])) + wave_u * 4096u;
    const uint32_t dstB = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sB[0][0])) + wave_u * 4096u;
    auto copy_a = [&](int t, int i) {
        __builtin_amdgcn_global_load_lds(DG_GLB(srcA[i] + (size_t)t * BK),
                                         DG_LDS_AT(dstA + (uint32_t)(t % S) * STAGE_BYTES + i * 1024u), 16, 0, 0);
    };
    auto copy_b = [&](int t, int i) {
        __builtin_amdgcn_global_load_lds(DG_GLB(srcB[i] + (size_t)t * kstepB),
                                         DG_LDS_AT(dstB + (uint32_t)(t % S) * STAGE_BYTES + i * 1024u), 16, 0, 0);
    };

    // ---- fragment addresses (bytes within a stage).
    // Q (A rows wm*128 + 32i + l32), P of column-major B (B rows wn*128 + 32j + l32):
    // lane holds k 8*lh .. 8*lh+7 of the step, chunk (2ks + lh) ^ ((l32 >> 2) & 3);
    // subtile i adds 32 rows = 2048 bytes.
    const int qsw = (l32 >> 2) & 3;
    int qoff[2], poff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        qoff[ks] = (wm * 128 + l32) * 64 + (((ks * 2 + lh) ^ qsw) << 4);
        poff[ks] = (wn * 128 + l32) * 64 + (((ks * 2 + lh) ^ qsw) << 4);
    }
    // P of row-major B (transpose reads): in each 16-lane group, lane i addresses k row
    // kb + i/4 at columns nb + 4(i%4) and receives column nb + i of rows kb..kb+3.
    // Lane groups 0/1 (2/3) cover columns 0-15 / 16-31 of k rows 0-7 (8-15) of the
    // step; step ks and half hh add (16 ks + 4 hh) rows of 512 bytes as immediates.
    int toff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = wn * 128 + j * 32 + (lg & 1) * 16 + ((l16 & 3) << 2);
        const int krow = (lg >> 1) * 8 + (l16 >> 2);
        toff[j] = krow * 512 + (((col >> 3) ^ nmaj32_swz(krow)) << 4) + (col & 7) * 2;
    }
    const uint32_t sA_base = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sA[0][0]));
    const uint32_t sB_base = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sB[0][0]));

    // One fragment set: q[i] (A), p[j] (B) as 8 halfs per lane; ph[j][hh] are the two
    // transpose-read halves of p[j] for row-major B.
    struct Frags {
        u32x4 q[4];
        u32x4 p[4];
        u32x2 ph[4][2];
    };
    Frags f0, f1;

    // Read the fragments of step ks of the tile in stage st into f, one read per call
    // position r (0..11): 4 Q reads, then 8 (row-major B) or 4 (column-major B) P reads.
    auto read_one = [&](Frags& f, int st, int ks, int r) {
        if (r < 4) {
            f.q[r] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sA[0][0]) + st * STAGE_BYTES +
                                                     qoff[ks] + r * 2048);
        } else if (OPB == 1) {
            if (r < 8)
                f.p[r - 4] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sB[0][0]) +
                                                            st * STAGE_BYTES + poff[ks] + (r - 4) * 2048);
        } else {
            const int j = (r - 4) >> 1, hh = (r - 4) & 1;
            const uint32_t addr = sB_base + (uint32_t)(st * STAGE_BYTES + toff[j] + (ks * 16 + hh * 4) * 512);
            asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.ph[j][hh]) : "v"(addr));
        }
    };
    constexpr int NREAD = OPB == 0 ? 12 : 8;
    // After the lgkmcnt(0) wait that ends a step: the transpose halves (asm outputs the
    // compiler cannot see being written late) pass through an empty asm placed after
    // the wait, so their uses cannot move above it; then they are joined into p[j].
    auto settle = [&](Frags& f) {
        if (OPB == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                asm volatile("" : "+v"(f.ph[j][0]), "+v"(f.ph[j][1]));
                f.p[j] = u32x4{f.ph[j][0][0], f.ph[j][0][1], f.ph[j][1][0], f.ph[j][1][1]};
            }
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    auto mfma = [&](const Frags& f, int i, int j) {
        if (DT == DT_F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, f.p[j]),
                                                               __builtin_bit_cast(f16x8, f.q[i]), acc[i][j], 0, 0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.p[j]),
                                                                __builtin_bit_cast(bf16x8, f.q[i]), acc[i][j], 0, 0, 0);
    };

    // One step: 16 MFMAs from `cur`, each followed by at most two other instructions
    // in a fixed order: the fragment reads of `nxt` two at a time after the first
    // MFMAs (early, so they are done by the wait that ends the step), then the four
    // copies of tile `ct` (half `half`: 0 = A, 1 = B) after every other MFMA of the
    // second half.
    auto step = [&](const Frags& cur, Frags& nxt, int rst, int rks, bool do_copy, int ct, int half) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            mfma(cur, k >> 2, k & 3);
            if (2 * k < NREAD) read_one(nxt, rst, rks, 2 * k);
            if (2 * k + 1 < NREAD) read_one(nxt, rst, rks, 2 * k + 1);
            if (do_copy && k >= 8 && (k & 1) == 0) {
                if (half == 0) copy_a(ct, (k - 8) >> 1);
                else copy_b(ct, (k - 8) >> 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: tiles 0, 1, 2 in flight (A then B of each); tile 0 complete; step (0, 0)
    // fragments read.
    for (int t = 0; t < D && t < nk; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) copy_a(t, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) copy_b(t, i);
    }
    vm_wait(8 * (min(D, nk) - 1));
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_one(f0, 0, 0, r);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(f0);

    // One iteration (tile t). REFILL: tile t+D exists and is copied. The reads of step
    // (t+1, 0) in the last iteration fetch a stage nobody writes any more; their values
    // are never used (this keeps the step free of branches).
    auto iteration = [&](int t, auto refill_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;
        const int st = t % S;
        // step (t, 0): MFMAs from f0; read step (t, 1) into f1; copy A of tile t+D
        step(f0, f1, st, 1, REFILL, t + D, 0);
        // own reads done; own copies of tile t+1 done (those of tiles t+2 .. t+D-1 and
        // the A half of tile t+D may still be in flight); then the barrier
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (REFILL) vm_wait_n<8 * (D - 2) + 4>();
        else vm_wait(8 * max(0, nk - t - 2));
        asm volatile("s_barrier" ::: "memory");
        settle(f1);
        // step (t, 1): MFMAs from f1; read step (t+1, 0) into f0; copy B of tile t+D
        step(f1, f0, (t + 1) % S, 0, REFILL, t + D, 1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        settle(f0);
    };
    int t = 0;
    for (; t + D < nk; ++t) iteration(t, std::true_type{});
    for (; t < nk; ++t) iteration(t, std::false_type{});

    // The empty asm below stands between the MFMAs and the reads of their results, so
    // the compiler's hazard padding does not see the MFMA as the last writer: the 18
    // wait states a 16-pass MFMA result needs before other instructions read it are
    // given here.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
    // plain stores: register r of subtile (i, j) holds C row m = wm*128 + 32i + l32,
    // columns n = wn*128 + 32j + 8(r/4) + 4*lh + r%4, i.e. four runs of 4 columns.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + l32;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // one subtile at a time: the empty asm pins acc[i][j] in the accumulation
            // registers until here (otherwise every accumulator is copied out up front,
            // which needs more registers than exist)
            asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = n0 + wn * 128 + j * 32 + rg * 8 + lh * 4;
                store_run4<false>(g, m, n, f32x4{acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2],
                                                 acc[i][j][4 * rg + 3]});
            }
        }
    }
}

}  // namespace dg
