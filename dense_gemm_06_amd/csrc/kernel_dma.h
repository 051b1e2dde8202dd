// kernel_dma.h -- software-pipelined MFMA kernel with direct global -> LDS copies.
#pragma once
#include <type_traits>

#include "lds_layout.h"

namespace dg {

// Software-pipelined MFMA kernel for 16-bit inputs on full 256 x 256 tiles (M and
// N multiples of 256, K a multiple of 32, 16-byte aligned operands).
//
// All 8 waves (2 x 4, 128 x 64 each, two per SIMD) multiply. The k loop runs in
// steps of 16 (one v_mfma_f32_32x32x16 per 32 x 32 subtile); the fragments of
// step s+1 are read from LDS while the 8 MFMAs of step s execute (two register
// sets). Tiles of k = 32 reach LDS through direct copies issued four tiles ahead
// into a ring of 4 stages, and one barrier per tile publishes the next tile and
// retires the stage just read.
//
// Tile t sits in stage t mod 4. Its fragments are read in steps 2t-1 (k 0..15)
// and 2t (k 16..31). The barrier between steps 2t and 2t+1 requires tile t+1 to
// be complete (each wave waits for its own copies of it; copies of tiles t+2 and
// t+3 may still be in flight) and all reads of stage t mod 4 done; right after
// it, tile t+4 is copied into that stage.
//
// On this chip the matrix unit and the rest of a SIMD's instruction stream do
// not overlap well, so the loop is kept short: the loop is unrolled once per
// stage so every fragment read is a fixed per-lane base plus an immediate
// offset, and the copies are issued from scalar base addresses. The copies are
// inline asm, which keeps them out of the compiler's view: it would otherwise
// wait for every in-flight copy before each LDS read. Their completion is
// waited for explicitly (vmcnt) before the barrier that publishes a tile.
template <int DT, int OPB>
__global__ __launch_bounds__(512) void mfma16_dma(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BK = 32, S = 4;
    constexpr int SA = BM * BK, SB = BN * BK;  // halfs per stage (16 KB each)
    __shared__ __attribute__((aligned(1024))) uint16_t sA[S * SA];
    __shared__ __attribute__((aligned(1024))) uint16_t sB[S * SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // wave tile rows wm*128.., columns wn*64..
    const int l32 = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = g.K / BK;

    // ---- copies: waves 0-3 copy the A tile, waves 4-7 the B tile; 4 blocks of 1 KB
    // each per wave. Lane L of block b lands at LDS byte b*1024 + 16L and loads the
    // logical 16-byte chunk that belongs at that swizzled position.
    const bool copiesA = wm == 0;
    const bool kmajor = copiesA || OPB == 1;
    uint32_t voff[4];  // per-lane byte offset from the wave-uniform global base
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = wn * 4 + i;
        if (kmajor) {
            const int row = b * 16 + (lane >> 2);
            const int c = (lane & 3) ^ kmaj32_swz(row);
            voff[i] = (uint32_t)(row * (copiesA ? g.lda : g.ldb) + c * 8) * 2u;
        } else {
            const int row = b * 2 + (lane >> 5);
            const int c = (lane & 31) ^ nmaj32_swz(row);
            voff[i] = (uint32_t)(row * g.ldb + c * 8) * 2u;
        }
    }
    const uint64_t gbase = copiesA ? reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(g.A) + (size_t)m0 * g.lda)
                           : OPB == 0 ? reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(g.B) + n0)
                                      : reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(g.B) + (size_t)n0 * g.ldb);
    const uint64_t gstep = (!copiesA && OPB == 0) ? (uint64_t)BK * g.ldb * 2u : (uint64_t)BK * 2u;  // bytes per k-tile
    const uint32_t ldsdst = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(copiesA ? sA : sB)) + (uint32_t)(wn * 4) * 1024u;
    // wave-uniform values, moved to scalar registers (the compiler cannot prove a
    // value derived from threadIdx.x / 64 is uniform). readfirstlane returns a signed
    // int: each half goes through uint32_t before widening, or a low word with bit 31
    // set would sign-extend into the high word of the address.
    auto uniform64 = [](uint64_t v) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | (uint64_t)lo;
    };
    const uint64_t gb = uniform64(gbase);
    const uint64_t gs = uniform64(gstep);
    const uint32_t ld0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)ldsdst);
    auto issue = [&](int t) {
        const uint64_t gp = gb + (uint64_t)t * gs;
        const uint32_t d = ld0 + (uint32_t)(t & 3) * (SA * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            // An SALU write of M0 needs one wait state before an LDS DMA reads it; the
            // compiler's hazard pass does not look inside asm, so the nop is explicit.
            // M0 is not declared clobbered (the compiler reserves it); no other code in
            // this kernel reads M0.
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff[i]),
                         "s"(d + i * 1024u), "s"(gp)
                         : "memory");
    };

    // ---- fragment reads: per-lane bases; subtile, k step and stage are immediates.
    // Q (A rows): k-major 64-byte rows, chunk (ks*2 + lane/32) ^ kmaj32_swz(row); the
    // swizzle depends on the lane only (rows differ by multiples of 32 between
    // subtiles), so one base per k step.
    const char* sAb = reinterpret_cast<const char*>(sA);
    const char* sBb = reinterpret_cast<const char*>(sB);
    const char* qb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int r = wm * 128 + l32;
        qb[ks] = sAb + r * 64 + (((ks * 2 + lh) ^ kmaj32_swz(r)) << 4);
    }
    // P (B columns): row-major B through transpose reads (4 consecutive k of one n per
    // lane), or column-major B like Q.
    const char* pbase[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (OPB == 0) {
            const int gp = lane >> 4, i16 = lane & 15;
            const int col = wn * 64 + j * 32 + (gp & 1) * 16 + ((i16 & 3) << 2);
            const int krow = (gp >> 1) * 8 + (i16 >> 2);  // ks*16 and hh*4 rows are added as immediates
            pbase[j][0] = sBb + krow * 512 + ((((col >> 3) ^ nmaj32_swz(krow))) << 4) + (col & 7) * 2;
            pbase[j][1] = nullptr;
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int r = wn * 64 + j * 32 + l32;
                pbase[j][ks] = sBb + r * 64 + (((ks * 2 + lh) ^ kmaj32_swz(r)) << 4);
            }
        }
    }

    u32x4 qa[2][4], pb[2][2];
    auto load_frags = [&](int f, auto stage_c, int ks) {
        constexpr int st = decltype(stage_c)::value;
        constexpr int so = st * SA * 2;  // stage offset in bytes
#pragma unroll
        for (int i = 0; i < 4; ++i)
            qa[f][i] = *DG_LDS_PTR(const u32x4, qb[ks] + so + i * 32 * 64);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (OPB == 0) {
                const char* p = pbase[j][0] + so + ks * 16 * 512;
                u32x2 h0, h1;
                if (DT == DT_F16) {
                    h0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(DG_LDS_PTR(fp16x4_t, p)));
                    h1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(DG_LDS_PTR(fp16x4_t, p + 4 * 512)));
                } else {
                    h0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DG_LDS_PTR(bf16x4_t, p)));
                    h1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DG_LDS_PTR(bf16x4_t, p + 4 * 512)));
                }
                pb[f][j] = u32x4{h0[0], h0[1], h1[0], h1[1]};
            } else {
                pb[f][j] = *DG_LDS_PTR(const u32x4, pbase[j][ks] + so);
            }
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto mma = [&](int f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (DT == DT_F16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, pb[f][j]),
                                                                      __builtin_bit_cast(f16x8, qa[f][i]), acc[i][j],
                                                                      0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pb[f][j]),
                                                                       __builtin_bit_cast(bf16x8, qa[f][i]), acc[i][j],
                                                                       0, 0, 0);
            }
    };
    auto tile_barrier = [&](int vm_allowed) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (vm_allowed >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else if (vm_allowed >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (vm_allowed >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // One tile t (stage ST = t mod 4): step 2t multiplies set 0 while reading k 16..31
    // of tile t into set 1; after the barrier, step 2t+1 multiplies set 1 while reading
    // k 0..15 of tile t+1 into set 0.
    auto tile = [&](auto st_c, int t) {
        constexpr int st = decltype(st_c)::value;
        using NEXT = std::integral_constant<int, (st + 1) & 3>;
        load_frags(1, st_c, 1);
        mma(0);
        tile_barrier(4 * max(0, min(2, nk - 2 - t)));
        if (t + S < nk) issue(t + S);
        load_frags(0, NEXT{}, 0);
        mma(1);
    };

    // prologue: tiles 0..3 in flight, tile 0 published, first fragments requested
    for (int t = 0; t < S && t < nk; ++t) issue(t);
    tile_barrier(4 * (min(S, nk) - 1));
    load_frags(0, I0{}, 0);

    int t = 0;
    for (; t + 4 <= nk - 1; t += 4) {
        tile(I0{}, t);
        tile(I1{}, t + 1);
        tile(I2{}, t + 2);
        tile(I3{}, t + 3);
    }
    // remaining tiles before the last one (t is a multiple of 4 here)
    if (t < nk - 1) {
        tile(I0{}, t);
        ++t;
        if (t < nk - 1) {
            tile(I1{}, t);
            ++t;
            if (t < nk - 1) {
                tile(I2{}, t);
                ++t;
            }
        }
    }
    // last tile (stage (nk-1) mod 4): no further copies or barriers
    switch ((nk - 1) & 3) {
        case 0: load_frags(1, I0{}, 1); break;
        case 1: load_frags(1, I1{}, 1); break;
        case 2: load_frags(1, I2{}, 1); break;
        default: load_frags(1, I3{}, 1); break;
    }
    mma(0);
    mma(1);

    // epilogue: lane owns C[m][n..n+3] for four n runs per subtile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + l32;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = n0 + wn * 64 + j * 32 + rg * 8 + lh * 4;
                store_run4<false>(g, m, n, f32x4{acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2],
                                                 acc[i][j][4 * rg + 3]});
            }
    }
}

}  // namespace dg
