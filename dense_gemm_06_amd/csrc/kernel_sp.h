// kernel_sp.h -- software-pipelined 32x32x16 MFMA kernel with direct LDS copies.
#pragma once
#include <type_traits>

#include "lds_layout.h"
#include "streamk.h"

// An LDS pointer made from a byte address (an integer): it carries no link to the
// LDS variable the address falls in.
#define DG_LDS_AT(a) ((__attribute__((address_space(3))) void*)(uintptr_t)(uint32_t)(a))

namespace dg {

// Wait until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ __forceinline__ void vm_wait_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same for a run-time even n in 0..24 (larger values wait for everything).
__device__ __forceinline__ void vm_wait(int n) {
    switch (n) {
        case 0: vm_wait_n<0>(); break;
        case 2: vm_wait_n<2>(); break;
        case 4: vm_wait_n<4>(); break;
        case 6: vm_wait_n<6>(); break;
        case 8: vm_wait_n<8>(); break;
        case 10: vm_wait_n<10>(); break;
        case 12: vm_wait_n<12>(); break;
        case 16: vm_wait_n<16>(); break;
        case 20: vm_wait_n<20>(); break;
        case 24: vm_wait_n<24>(); break;
        default: vm_wait_n<0>(); break;
    }
}

// The first v (0..8) of a chunk of eight 16-bit elements, the rest zero, from w =
// the 8 elements that END at the chunk's last valid one (element j of w is element
// j - (8 - v) of the chunk): w shifted down by 8 - v elements as a 128-bit value.
__device__ __forceinline__ u32x4 keep_first8(u32x4 w, int v) {
    if (v >= 8) return w;
    if (v <= 0) return u32x4{0, 0, 0, 0};
    const uint64_t lo = ((uint64_t)w[1] << 32) | w[0], hi = ((uint64_t)w[3] << 32) | w[2];
    const int s = 16 * (8 - v);  // 16 .. 112 bits
    uint64_t olo, ohi;
    if (s >= 64) {
        olo = hi >> (s - 64);
        ohi = 0;
    } else {
        olo = (lo >> s) | (hi << (64 - s));
        ohi = hi >> s;
    }
    return u32x4{(uint32_t)olo, (uint32_t)(olo >> 32), (uint32_t)ohi, (uint32_t)(ohi >> 32)};
}

// Software-pipelined MFMA kernel for 16-bit inputs on 256 x 256 tiles (K a multiple
// of 8, 16-byte aligned operands; edge tiles in M, and in N for column-major B or for
// N a multiple of 8, and a partial last k-tile, are handled as described below).
//
// NW = 4: four waves, one per SIMD, each owning a 128 x 128 quarter of the tile with
// its 16 v_mfma_f32_32x32x16 accumulators (256 registers) in the accumulation
// registers. NW = 8: eight waves, two per SIMD, each owning 128 x 64 (8
// accumulators). A 128 x 128 wave reads 64 bytes of LDS fragments per 32x32x16
// MFMA, a 128 x 64 wave 96; a single wave issues this instruction at about 87% of
// the matrix unit's rate, two waves per SIMD near 100%.
//
// The k loop runs in steps of 16. Each wave holds two fragment sets: while the
// MFMAs of step s run from one set, the fragment reads of step s+1 fill the other,
// interleaved with the MFMAs. Tiles of k = 32 (two steps) arrive by direct global
// -> LDS copies (global_load_lds_dwordx4) into a ring of 4 stages, issued three
// tiles ahead: each wave copies its share of the A tile during the first step of a
// tile and of the B tile during the second. One barrier per tile, between its two
// steps, makes the next tile visible (each wave first waits for its own copies of
// it) and retires the stage the refill of the current iteration overwrites.
//
// Tile t sits in stage t mod 4. Step (t, 0)'s fragments are read during step
// (t-1, 1), step (t, 1)'s during step (t, 0). The last reads of stage t mod 4 are
// therefore done (lgkmcnt(0)) before the barrier of iteration t, and iteration
// t+1 refills that stage with tile t+4.
//
// LDS layouts and the fragment maps are those of the 32x32x16 ping-pong form:
// k-major 64-byte rows with chunk swizzle kmaj32_swz, row-major B with nmaj32_swz,
// read through ds_read_b64_tr_b16. Both swizzles depend on the lane only for the
// rows a wave reads, so every fragment read is a per-lane base plus an immediate.
//
// Epilogue: the accumulators go through the LDS the k loop no longer needs, half
// a wave tile at a time (64 rows), and leave as whole rows: each store instruction
// writes 2 (NW = 4) or 4 (NW = 8) rows of the wave tile, contiguous in C. A fused
// epilogue (ep.kind != 0) is applied on the way out.
//
// REG = true is the same kernel for operands that are only aligned to their element
// (rows at any 2-byte offset) and for any K >= 8 and any N >= 8: each 16-byte chunk
// a lane owns goes global -> registers -> LDS instead of straight into LDS. Every
// chunk is exactly one 16-byte load, from an address inside the row (a chunk that
// straddles K, or N for a row-major B, is loaded as the 8 elements that end at the
// row's last valid one and shifted into place, zero-filled, when written; a chunk
// wholly past the end is loaded from the row start and written as zeros), so the
// load counter always counts 2*CPB loads per tile and wave. Tile t+1 is written to
// its stage during step (t, 0), before the barrier that publishes it, from registers
// loaded one iteration earlier; the load of tile t+2 then reuses them. The LDS
// layout, the fragment reads, the MFMAs and the epilogue are those of the direct-copy
// form.
//
// STREAM-K (persistent direct-copy form, g.sk_tiles > 0): after its whole rounds of
// tiles each of the first g.sk_width workgroups takes its share of the tail tiles'
// k-tiles (streamk.h), as at most two pieces, each a tile with its own k range and
// k-tile count (at least 4, so the copy stream carries over between pieces as
// between tiles). A piece that does not cover its tile stores its partial sum, as
// plain fp32, to its workspace slot; the fixup launch completes those tiles.
//
// GROUPED (persistent direct-copy form only): the tiles are those of a grouped call's
// problems, in the linear order of its segment table (each problem, batch member and
// tile raster as for the register-staged grouped kernels); each tile carries its own
// operands, leading dimensions, M, N, K and C, and the copy stream runs on across
// problems as across tiles. g then holds only xcd_remap (and no fused epilogue).
template <int DT, int OPB, int NW, bool REG, bool PERSIST, bool GROUPED>
__device__ __forceinline__ void mfma32_sp_body(GemmArgs& g, const GroupArgs* ga) {
    static_assert(NW == 4 || NW == 8, "waves");
    static_assert(!GROUPED || (PERSIST && !REG && NW == 8), "grouped: the persistent direct-copy form");
    constexpr int BM = 256, BN = 256, BK = 32, S = 4, D = S - 1;  // D: copy distance in tiles
    constexpr int SA = BM * BK, SB = BN * BK;                     // halfs per stage
    constexpr int STAGE_BYTES = SA * 2;                           // 16 KB for each of A and B
    constexpr int WNN = NW / 2;                                   // waves along n
    constexpr int SJ = 8 / WNN;                                   // 32-column subtiles per wave
    constexpr int CPB = 16 / NW;                                  // 1 KB copies per wave and operand
    __shared__ __attribute__((aligned(1024))) uint16_t sA[S][SA];
    __shared__ __attribute__((aligned(1024))) uint16_t sB[S][SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WNN, wn = wave % WNN;
    const int l32 = lane & 31, lh = lane >> 5;
    const int l16 = lane & 15, lg = lane >> 4;
    // Output tiles: one per workgroup (grid = tiles) or, for the direct-copy form, a
    // persistent grid that takes them in rounds of its size (the tile loop below).
    // With xcd_remap each XCD's workgroups take a contiguous run of each round.
    int tiles_total;
    if constexpr (GROUPED) tiles_total = ga->total_tiles;
    else tiles_total = g.tiles_m * g.tiles_n;
    // A unit of work: tile `tile` over k-tiles kb .. kb + nk - 1 (nk < 0: all of its
    // problem's K), its sum stored to C (slot < 0) or to workspace slot `slot`.
    struct Unit {
        int tile, kb, nk, slot;
    };
    // Unit u of this workgroup: round u of the whole tiles, then (stream-K) the pieces
    // of its share of the tail; false past the last one.
    const int sk_tiles = (PERSIST && !GROUPED) ? g.sk_tiles : 0;
    const int dp_total = tiles_total - sk_tiles;  // a multiple of the grid when sk_tiles > 0
    const int dp_rounds = sk_tiles > 0 ? dp_total / (int)gridDim.x : 0;
    auto unit_at = [&](int u, Unit& un) -> bool {
        un.kb = 0;
        un.nk = -1;
        un.slot = -1;
        if (sk_tiles == 0 || u < dp_rounds) {
            un.tile = round_tile(u, sk_tiles > 0 ? dp_total : tiles_total, g.xcd_remap);
            return un.tile >= 0;
        }
        // the shares go to hardware ids 0 .. sk_width - 1, which the dispatcher
        // spreads round-robin over the XCDs
        const int kt = (g.K + BK - 1) / BK;
        const int w = (int)blockIdx.x, p = u - dp_rounds;
        int t, kb, nk;
        if (w >= g.sk_width || p > 1 || !sk_piece(w, p, g.sk_width, sk_tiles, kt, t, kb, nk)) return false;
        un.tile = dp_total + t;
        un.kb = kb;
        un.nk = nk;
        un.slot = nk == kt ? -1 : 2 * w + p;
        return true;
    };
    int round = 0;
    Unit first;
    if constexpr (PERSIST) {
        // a stream-K share can be empty: the whole workgroup leaves before its first barrier
        if (!unit_at(0, first)) return;
    } else {
        first.tile = round_tile(0, tiles_total, g.xcd_remap);
        first.kb = 0;
        first.nk = -1;
        first.slot = -1;
    }
    // K a multiple of 8: the last k-tile may be partial (krem of its 32 k valid); its
    // copies clamp the chunks at or beyond K and the LDS chunks past K are zeroed
    // before any fragment of that tile is read
    const int nk = (g.K + BK - 1) / BK;
    const int krem = g.K - (nk - 1) * BK;
    const bool ktail = krem < BK;

    // ---- direct copies: wave w moves blocks CPB*w .. CPB*w+CPB-1 (1 KB each) of the A
    // tile and of the B tile. Lane L of block b lands at LDS byte b*1024 + 16L, a fixed
    // swizzled position, and loads the logical 16-byte chunk that belongs there.
    // Edge tiles (M or N not a multiple of 256): rows of A, and of a column-major B,
    // at or beyond M (N) copy row M - 1 (N - 1) instead, and 16-byte column chunks of
    // a row-major B that start at or beyond N copy columns 0..7 (N is then a multiple
    // of 8, so no chunk straddles N); what they bring in only reaches rows and
    // columns of C that the epilogue does not store.
    // kcA / kcB: the k offset of a lane's chunk within the k-tile (k-major copies);
    // krB: the k row of a lane's chunk (row-major B). A lane whose chunk of the last
    // tile starts at or beyond K copies the chunk at k = 0 of its row instead.
    int kcA[CPB], kcB[CPB];
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
        const int b = wave * CPB + i;
        const int row = b * 16 + (lane >> 2);
        kcA[i] = ((lane & 3) ^ kmaj32_swz(row)) << 3;
        kcB[i] = OPB == 1 ? kcA[i] : b * 2 + (lane >> 5);
    }
    // A lane's chunk sources for one output tile, the tile's origin, and what the tile
    // needs of its problem: the k-tile count, the step between k-tiles of B, and C
    // with its leading dimension and bounds (the call's, or the tile's problem's in a
    // grouped call).
    struct Src {
        const uint16_t* a[CPB];
        const uint16_t* b[CPB];
        int nv[CPB];  // REG, row-major B: columns of the lane's chunk inside N (0..8)
        int m0, n0;
        int M, N, nk;
        size_t kstep_b;  // elements per k-tile of B
        float* C;        // element (m, n) at C[m * ldc + n]
        int64_t ldc;
        bool plain;      // a partial sum for the workspace: no fused epilogue
    };
    // The problem of tile t: operands, leading dimensions, sizes and tile coordinates.
    struct Prob {
        const uint16_t* A;
        const uint16_t* B;
        float* C;
        int64_t lda, ldb, ldc;
        int M, N, K, tm, tn;
    };
    auto prob_of = [&](int t, Prob& p) {
        if constexpr (GROUPED) {
            GemmArgs gt;
            group_tile<2>(*ga, t, gt, p.tm, p.tn);
            p.A = static_cast<const uint16_t*>(gt.A);
            p.B = static_cast<const uint16_t*>(gt.B);
            p.C = gt.C;
            p.lda = gt.lda;
            p.ldb = gt.ldb;
            p.ldc = gt.ldc;
            p.M = gt.M;
            p.N = gt.N;
            p.K = gt.K;
        } else {
            raster(t, g.tiles_m, g.tiles_n, g.group_m, p.tm, p.tn);
            p.A = static_cast<const uint16_t*>(g.A);
            p.B = static_cast<const uint16_t*>(g.B);
            p.C = g.C;
            p.lda = g.lda;
            p.ldb = g.ldb;
            p.ldc = g.ldc;
            p.M = g.M;
            p.N = g.N;
            p.K = g.K;
        }
    };
    auto make_src = [&](const Unit& un, Src& s) {
        Prob p;
        prob_of(un.tile, p);
        s.m0 = p.tm * BM;
        s.n0 = p.tn * BN;
        s.M = p.M;
        s.N = p.N;
        s.nk = un.nk < 0 ? (p.K + BK - 1) / BK : un.nk;
        s.kstep_b = OPB == 0 ? (size_t)BK * p.ldb : (size_t)BK;
        s.plain = un.slot >= 0;
        if (un.slot >= 0) {
            // the slot holds the tile at leading dimension BN: element (m, n) of C
            // lands at slot[(m - m0) * BN + n - n0]
            s.C = g.work + ((ptrdiff_t)un.slot * (BM * BN) - ((ptrdiff_t)s.m0 * BN + s.n0));
            s.ldc = BN;
        } else {
            s.C = p.C;
            s.ldc = p.ldc;
        }
        // the unit's first k (0 unless it is a stream-K piece)
        const size_t k0 = (size_t)un.kb * BK;
#pragma unroll
        for (int i = 0; i < CPB; ++i) {
            const int b = wave * CPB + i;
            const int row = b * 16 + (lane >> 2);
            s.a[i] = p.A + (size_t)min(s.m0 + row, p.M - 1) * p.lda + k0 + kcA[i];
            if (OPB == 1) {
                s.b[i] = p.B + (size_t)min(s.n0 + row, p.N - 1) * p.ldb + k0 + kcB[i];
            } else {
                const int krow = kcB[i];  // k row within the k-tile
                const int col = s.n0 + (((lane & 31) ^ nmaj32_swz(krow)) << 3);
                const size_t kr = k0 + (size_t)krow;
                if constexpr (REG) {
                    // a chunk that straddles N is read from the row's last 8 columns, one
                    // wholly past N from column 0 (N >= 8); the write shifts or zeroes it
                    const int v = p.N - col;
                    s.nv[i] = v < 0 ? 0 : (v > 8 ? 8 : v);
                    s.b[i] = p.B + kr * p.ldb + (v >= 8 ? col : v > 0 ? p.N - 8 : 0);
                } else {
                    s.b[i] = p.B + kr * p.ldb + (col < p.N ? col : 0);
                }
            }
        }
    };
    Src cur;  // the tile being computed
    make_src(first, cur);
    // LDS destinations as plain wave-uniform numbers (M0 takes them directly). Built
    // from an integer, a copy's LDS pointer carries no link to sA / sB, so the
    // compiler does not make every later LDS read wait for all copies in flight
    // (vmcnt(0)); the explicit waits below order them instead.
    const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    const uint32_t dstA = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sA[0][0])) + wave_u * (CPB * 1024u);
    const uint32_t dstB = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sB[0][0])) + wave_u * (CPB * 1024u);
    // Copy chunk i of k-tile t of the tile whose sources are s into stage st (0..3).
    // TAIL: t is the partial last k-tile.
    auto copy_a = [&](const Src& s, int t, uint32_t st, int i, auto tail_tag) {
        const uint16_t* src = s.a[i] + (size_t)t * BK;
        if (decltype(tail_tag)::value && kcA[i] >= krem) src = s.a[i] - kcA[i];
        __builtin_amdgcn_global_load_lds(DG_GLB(src), DG_LDS_AT(dstA + st * STAGE_BYTES + i * 1024u), 16, 0, 0);
    };
    auto copy_b = [&](const Src& s, int t, uint32_t st, int i, auto tail_tag) {
        const uint16_t* src = s.b[i] + (size_t)t * s.kstep_b;
        if (decltype(tail_tag)::value && kcB[i] >= krem)
            src = OPB == 1 ? s.b[i] - kcB[i] : s.b[i] - (size_t)kcB[i] * g.ldb;
        __builtin_amdgcn_global_load_lds(DG_GLB(src), DG_LDS_AT(dstB + st * STAGE_BYTES + i * 1024u), 16, 0, 0);
    };
    // Zero the chunks of stage st that lie at or beyond K (the partial last tile), then
    // wait for this wave's writes; the caller's barrier publishes them.
    auto zero_tail = [&](int st) {
        char* sa = reinterpret_cast<char*>(&sA[st][0]);
        char* sb = reinterpret_cast<char*>(&sB[st][0]);
        for (int idx = tid; idx < BM * 4; idx += NW * 64) {
            const int r = idx >> 2, c = idx & 3;
            if (c * 8 >= krem) *reinterpret_cast<u32x4*>(sa + r * 64 + ((c ^ kmaj32_swz(r)) << 4)) = u32x4{0, 0, 0, 0};
        }
        if (OPB == 1) {
            for (int idx = tid; idx < BN * 4; idx += NW * 64) {
                const int r = idx >> 2, c = idx & 3;
                if (c * 8 >= krem)
                    *reinterpret_cast<u32x4*>(sb + r * 64 + ((c ^ kmaj32_swz(r)) << 4)) = u32x4{0, 0, 0, 0};
            }
        } else {
            // k rows krem .. 31 of 512 bytes each (the swizzle only permutes chunks within a row)
            for (int idx = krem * 32 + tid; idx < BK * 32; idx += NW * 64)
                *reinterpret_cast<u32x4*>(sb + idx * 16) = u32x4{0, 0, 0, 0};
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    // ---- register staging (REG). Tile t's chunks: ra (A) and rb (B), one 16-byte load
    // each; written to stage t & 3 at the LDS position the direct copy would fill.
    u32x4 ra[CPB], rb[CPB];
    const bool nedge = OPB == 0 && cur.n0 + BN > g.N;  // a row-major B tile that crosses N
    auto ld16 = [](const uint16_t* p) {
        u32x4 r;
        __builtin_memcpy(&r, p, 16);  // one global_load_dwordx4; gfx950 serves under-aligned ones
        return r;
    };
    // chunk c of tile t: c < CPB is A chunk c, else B chunk c - CPB. TAIL: t is the
    // partial last k-tile.
    auto load_reg = [&](int t, int c, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        if (c < CPB) {
            const uint16_t* src = cur.a[c] + (size_t)t * BK;
            if (TAIL) {
                const int v = g.K - (t * BK + kcA[c]);
                if (v < 8) src = cur.a[c] - kcA[c] + (v > 0 ? g.K - 8 : 0);
            }
            ra[c] = ld16(src);
        } else {
            const int i = c - CPB;
            const uint16_t* src = cur.b[i] + (size_t)t * cur.kstep_b;
            if (TAIL) {
                if (OPB == 1) {
                    const int v = g.K - (t * BK + kcB[i]);
                    if (v < 8) src = cur.b[i] - kcB[i] + (v > 0 ? g.K - 8 : 0);
                } else if (t * BK + kcB[i] >= g.K) {
                    src = cur.b[i] + (size_t)(g.K - 1 - kcB[i]) * g.ldb;  // row K - 1, written as zeros
                }
            }
            rb[i] = ld16(src);
        }
    };
    auto write_reg = [&](int t, int c, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        u32x4 v;
        uint32_t addr;
        if (c < CPB) {
            v = ra[c];
            if (TAIL) v = keep_first8(v, g.K - (t * BK + kcA[c]));
            addr = dstA + (uint32_t)(t & 3) * STAGE_BYTES + (uint32_t)c * 1024u;
        } else {
            const int i = c - CPB;
            v = rb[i];
            if (OPB == 1) {
                if (TAIL) v = keep_first8(v, g.K - (t * BK + kcB[i]));
            } else {
                if (nedge) v = keep_first8(v, cur.nv[i]);
                if (TAIL && t * BK + kcB[i] >= g.K) v = u32x4{0, 0, 0, 0};
            }
            addr = dstB + (uint32_t)(t & 3) * STAGE_BYTES + (uint32_t)i * 1024u;
        }
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(DG_LDS_AT(addr + (uint32_t)lane * 16u)) = v;
    };

    // ---- fragment addresses (bytes within a stage).
    // Q (A rows wm*128 + 32i + l32), P of column-major B (B rows wn*32*SJ + 32j + l32):
    // lane holds k 8*lh .. 8*lh+7 of the step, chunk (2ks + lh) ^ ((l32 >> 2) & 3);
    // a subtile adds 32 rows = 2048 bytes.
    const int qsw = (l32 >> 2) & 3;
    int qoff[2], poff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        qoff[ks] = (wm * 128 + l32) * 64 + (((ks * 2 + lh) ^ qsw) << 4);
        poff[ks] = (wn * 32 * SJ + l32) * 64 + (((ks * 2 + lh) ^ qsw) << 4);
    }
    // P of row-major B (transpose reads): in each 16-lane group, lane i addresses k row
    // kb + i/4 at columns nb + 4(i%4) and receives column nb + i of rows kb..kb+3.
    // Lane groups 0/1 (2/3) cover columns 0-15 / 16-31 of k rows 0-7 (8-15) of the
    // step; step ks and half hh add (16 ks + 4 hh) rows of 512 bytes as immediates.
    int toff[SJ];
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
        const int col = wn * 32 * SJ + j * 32 + (lg & 1) * 16 + ((l16 & 3) << 2);
        const int krow = (lg >> 1) * 8 + (l16 >> 2);
        toff[j] = krow * 512 + (((col >> 3) ^ nmaj32_swz(krow)) << 4) + (col & 7) * 2;
    }
    const uint32_t sB_base = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(&sB[0][0]));

    // One fragment set: q[i] (A), p[j] (B) as 8 halfs per lane; ph[j][hh] are the two
    // transpose-read halves of p[j] for row-major B.
    struct Frags {
        u32x4 q[4];
        u32x4 p[SJ];
        u32x2 ph[SJ][2];
    };
    Frags f0, f1;

    // Read number r of step ks of the tile in stage st into f: 4 Q reads, then 2*SJ
    // (row-major B) or SJ (column-major B) P reads.
    auto read_one = [&](Frags& f, int st, int ks, int r) {
        if (r < 4) {
            f.q[r] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sA[0][0]) + st * STAGE_BYTES +
                                                     qoff[ks] + r * 2048);
        } else if (OPB == 1) {
            f.p[r - 4] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sB[0][0]) +
                                                        st * STAGE_BYTES + poff[ks] + (r - 4) * 2048);
        } else {
            const int j = (r - 4) >> 1, hh = (r - 4) & 1;
            const uint32_t addr = sB_base + (uint32_t)(st * STAGE_BYTES + toff[j] + (ks * 16 + hh * 4) * 512);
            asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.ph[j][hh]) : "v"(addr));
        }
    };
    constexpr int NREAD = 4 + (OPB == 0 ? 2 * SJ : SJ);
    // After the lgkmcnt(0) wait that ends a step: the transpose halves (asm outputs the
    // compiler cannot see being written late) pass through an empty asm placed after
    // the wait, so their uses cannot move above it; then they are joined into p[j].
    auto settle = [&](Frags& f) {
        if (OPB == 0) {
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                asm volatile("" : "+v"(f.ph[j][0]), "+v"(f.ph[j][1]));
                f.p[j] = u32x4{f.ph[j][0][0], f.ph[j][0][1], f.ph[j][1][0], f.ph[j][1][1]};
            }
        }
    };

    f32x16 acc[4][SJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j) acc[i][j] = f32x16{};

    auto mfma = [&](const Frags& f, int i, int j) {
        if (DT == DT_F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, f.p[j]),
                                                               __builtin_bit_cast(f16x8, f.q[i]), acc[i][j], 0, 0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.p[j]),
                                                                __builtin_bit_cast(bf16x8, f.q[i]), acc[i][j], 0, 0, 0);
    };

    // One step: 4*SJ MFMAs from `cur`, each followed by at most two other instructions
    // in a fixed order: the fragment reads of `nxt` two at a time after the first
    // MFMAs (early, so they are done by the wait that ends the step), then this wave's
    // CPB copies of k-tile `ct` of the tile with sources `cs` into stage `cst` (half
    // `half`: 0 = A, 1 = B) after every other MFMA of the second half of the step.
    constexpr int NM = 4 * SJ;  // MFMAs per step
    auto step = [&](const Frags& cur_f, Frags& nxt_f, int rst, int rks, bool do_copy, const Src& cs, int ct,
                    uint32_t cst, int half, auto tail_tag) {
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            mfma(cur_f, k / SJ, k % SJ);
            if (2 * k < NREAD) read_one(nxt_f, rst, rks, 2 * k);
            if (2 * k + 1 < NREAD) read_one(nxt_f, rst, rks, 2 * k + 1);
            const int c = (k - NM / 2) >> 1;
            if (do_copy && k >= NM / 2 && (k & 1) == 0 && c < CPB) {
                if (half == 0) copy_a(cs, ct, cst, c, tail_tag);
                else copy_b(cs, ct, cst, c, tail_tag);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- epilogues. Before either, every wave's last fragment reads are done
    // (lgkmcnt(0) at the end of the last iteration) and a barrier makes sure all of
    // them are before any wave overwrites a stage. The empty asm before that barrier
    // stands between the MFMAs and the reads of their results, so the compiler's hazard
    // padding does not see the MFMA as the last writer: the 18 wait states a 16-pass
    // MFMA result needs are given here.
    const int wrow0 = wm * 128, wcol0 = wn * 32 * SJ;  // the wave's tile within the output tile
    auto store4 = [&](int m, int n, f32x4 v) {
        if (m < g.M) {
            if (g.ep.kind == 0) store_run4<false>(g, m, n, v);
            else epilogue_run4_body(g.ep, g.C, g.ldc, g.N, m, n, v);
        }
    };
    // The same for the persistent form, with C, its leading dimension and bounds from
    // the tile's sources (its own problem's in a grouped call, which has no fused
    // epilogue)
    auto store4p = [&](const Src& s, int m, int n, f32x4 v) {
        if (m >= s.M) return;
        if (GROUPED || g.ep.kind == 0 || s.plain) {
            float* cp = s.C + (size_t)m * s.ldc + n;
            if (n + 3 < s.N) {
                __builtin_memcpy(cp, &v, 16);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < s.N) cp[e] = v[e];
            }
        } else {
            epilogue_run4_body(g.ep, g.C, g.ldc, g.N, m, n, v);
        }
    };
    // The whole LDS, 64 rows of the wave tile at a time: each wave owns a slot of 64
    // rows x WT bytes (WT = 32*SJ fp32 = 512 or 256 bytes): NW = 4: 32 KB, waves 0-1 in
    // sA, 2-3 in sB; NW = 8: 16 KB, waves 0-3 in sA, 4-7 in sB. Register r of subtile
    // (i, j) holds row 32i + l32 of the wave tile and columns 32j + 8(r/4) + 4*lh + r%4:
    // chunk c = 8j + 2(r/4) + lh of 16 bytes, stored at position c ^ (row & 15) of its
    // row, which keeps both the writes (16 rows per lane phase) and the whole-row reads
    // free of bank conflicts; each store instruction writes 2 (NW = 4) or 4 (NW = 8)
    // whole rows of the wave tile, contiguous in C.
    auto full_epilogue = [&](const Src& s) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
        __syncthreads();
        constexpr int WT = 32 * SJ * 4;           // bytes per wave-tile row
        constexpr int CPR = WT / 16;              // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;             // rows per read instruction
        constexpr int SLOT = 64 * WT;
        char* slot = reinterpret_cast<char*>(wave < NW / 2 ? &sA[0][0] : &sB[0][0]) + (wave % (NW / 2)) * SLOT;
        const int cm0 = s.m0 + wrow0, cn0 = s.n0 + wcol0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * h + ii;
                const int row = ii * 32 + l32;
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    // one subtile at a time: the empty asm pins acc[i][j] in the accumulation
                    // registers until here (otherwise all accumulators are copied out at
                    // once, which needs more registers than exist)
                    asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int c = j * 8 + rg * 2 + lh;
                        *reinterpret_cast<f32x4*>(slot + row * WT + ((c ^ (row & 15)) << 4)) =
                            f32x4{acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
                    }
                }
            }
            // only this wave touches its slot; the wave barrier keeps the compiler from
            // moving LDS accesses across the write / read phases, which the hardware runs
            // in order within a wave
            __builtin_amdgcn_wave_barrier();
            for (int it = 0; it < 64 / RPI; ++it) {
                const int row = it * RPI + lane / CPR, c = lane % CPR;
                const f32x4 v = *reinterpret_cast<const f32x4*>(slot + row * WT + ((c ^ (row & 15)) << 4));
                store4(cm0 + h * 64 + row, cn0 + c * 4, v);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };

    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    if constexpr (REG) {
    // One step of the register-staged form: as `step`, with no copies; with a write
    // tag (tile wt exists), the second half of the step first waits for this wave's
    // loads of tile wt, then writes one chunk of it after each MFMA and, with a load
    // tag (tile lt exists), loads the same chunk of tile lt into the freed registers.
    auto step_reg = [&](const Frags& cur, Frags& nxt, int rst, int rks, int wt, int lt, auto write_tag,
                        auto load_tag) {
        constexpr int W = decltype(write_tag)::value, L = decltype(load_tag)::value;  // 0 none, 1 full, 2 tail
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            mfma(cur, k / SJ, k % SJ);
            if (2 * k < NREAD) read_one(nxt, rst, rks, 2 * k);
            if (2 * k + 1 < NREAD) read_one(nxt, rst, rks, 2 * k + 1);
            if constexpr (W != 0) {
                if (k >= NM / 2) {
                    const int c = k - NM / 2;  // chunk 0 .. 2*CPB - 1
                    if (c == 0) vm_wait_n<0>();
                    write_reg(wt, c, std::integral_constant<bool, W == 2>{});
                    if constexpr (L != 0) load_reg(lt, c, std::integral_constant<bool, L == 2>{});
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    constexpr std::integral_constant<int, 0> none{};
    constexpr std::integral_constant<int, 1> full{};
    constexpr std::integral_constant<int, 2> part{};
    // prologue: tile 0 loaded, written to stage 0; tile 1 loaded; step (0, 0)
    // fragments read.
    if (ktail && nk == 1) {
#pragma unroll
        for (int c = 0; c < 2 * CPB; ++c) load_reg(0, c, yes);
        vm_wait_n<0>();
#pragma unroll
        for (int c = 0; c < 2 * CPB; ++c) write_reg(0, c, yes);
    } else {
#pragma unroll
        for (int c = 0; c < 2 * CPB; ++c) load_reg(0, c, no);
        vm_wait_n<0>();
#pragma unroll
        for (int c = 0; c < 2 * CPB; ++c) write_reg(0, c, no);
    }
    if (nk > 1) {
        if (ktail && nk == 2) {
#pragma unroll
            for (int c = 0; c < 2 * CPB; ++c) load_reg(1, c, yes);
        } else {
#pragma unroll
            for (int c = 0; c < 2 * CPB; ++c) load_reg(1, c, no);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_one(f0, 0, 0, r);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(f0);
    // One iteration (tile t): step (t, 0) writes tile t+1 (tag W) and loads tile t+2
    // (tag L); the barrier publishes tile t+1; step (t, 1) reads step (t+1, 0).
    auto iteration_reg = [&](int t, auto write_tag, auto load_tag) {
        step_reg(f0, f1, t & 3, 1, t + 1, t + 2, write_tag, load_tag);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        settle(f1);
        step_reg(f1, f0, (t + 1) & 3, 0, 0, 0, none, none);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        settle(f0);
    };
    // straight runs of one variant each, as in the direct-copy form
    const int nfull = ktail ? nk - 1 : nk;  // whole k-tiles
    int t = 0;
    for (; t + 2 < nfull; ++t) iteration_reg(t, full, full);
    for (; ktail && t + 2 == nk - 1; ++t) iteration_reg(t, full, part);  // loads the partial tile
    for (; t + 2 < nk; ++t) iteration_reg(t, full, none);
    for (; ktail && t + 2 == nk; ++t) iteration_reg(t, part, none);      // writes the partial tile
    for (; t + 1 < nk; ++t) iteration_reg(t, full, none);
    for (; t < nk; ++t) iteration_reg(t, none, none);
    full_epilogue(cur);
    } else if constexpr (!PERSIST) {
    // ---- the direct-copy form, one output tile per workgroup.
    // prologue: k-tiles 0 .. D-1 in flight (A then B of each); k-tile 0 complete; step
    // (0, 0) fragments read.
    for (int t = 0; t < D && t < nk; ++t) {
        if (ktail && t == nk - 1) {
#pragma unroll
            for (int i = 0; i < CPB; ++i) copy_a(cur, t, (uint32_t)t, i, yes);
#pragma unroll
            for (int i = 0; i < CPB; ++i) copy_b(cur, t, (uint32_t)t, i, yes);
        } else {
#pragma unroll
            for (int i = 0; i < CPB; ++i) copy_a(cur, t, (uint32_t)t, i, no);
#pragma unroll
            for (int i = 0; i < CPB; ++i) copy_b(cur, t, (uint32_t)t, i, no);
        }
    }
    vm_wait(2 * CPB * (min(D, nk) - 1));
    asm volatile("s_barrier" ::: "memory");
    if (ktail && nk == 1) {
        zero_tail(0);
        asm volatile("s_barrier" ::: "memory");
    }
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_one(f0, 0, 0, r);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(f0);

    // One iteration (k-tile t, in stage t & 3). REFILL: k-tile t+D exists and is copied
    // (TAIL: it is the partial last k-tile). FIX: k-tile t+1 is the partial last tile,
    // whose chunks past K are zeroed between the barrier that completes its copies and
    // the first reads of it. The reads of step (t+1, 0) in the last iteration fetch a
    // stage nobody writes any more; their values are never used (this keeps the step
    // free of branches).
    auto iteration = [&](int t, auto refill_tag, auto tail_tag, auto fix_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;
        const int st = t & 3;
        // step (t, 0): MFMAs from f0; read step (t, 1) into f1; copy A of k-tile t+D
        step(f0, f1, st, 1, REFILL, cur, t + D, (uint32_t)((t + D) & 3), 0, tail_tag);
        // own reads done; own copies of k-tile t+1 done (those of k-tiles t+2 .. t+D-1
        // and the A half of k-tile t+D may still be in flight); then the barrier
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (REFILL) vm_wait_n<2 * CPB * (D - 2) + CPB>();
        else vm_wait(2 * CPB * max(0, nk - t - 2));
        asm volatile("s_barrier" ::: "memory");
        if (decltype(fix_tag)::value) {
            zero_tail((t + 1) & 3);
            asm volatile("s_barrier" ::: "memory");
        }
        settle(f1);
        // step (t, 1): MFMAs from f1; read step (t+1, 0) into f0; copy B of k-tile t+D
        step(f1, f0, (t + 1) & 3, 0, REFILL, cur, t + D, (uint32_t)((t + D) & 3), 1, tail_tag);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        settle(f0);
    };
    // straight runs of one variant each (a branch between two inlined variants inside
    // a loop leaves the register allocator unable to keep the fragments in registers)
    const int nfull = ktail ? nk - 1 : nk;  // k-tiles t + D copied by the plain variant
    int t = 0;
    for (; t + D < nfull; ++t) iteration(t, yes, no, no);
    for (; ktail && t + D == nk - 1; ++t) iteration(t, yes, yes, no);  // copies the partial tile
    const int nfix = ktail ? nk - 2 : nk;   // the iteration before the partial tile
    for (; t < nfix; ++t) iteration(t, no, no, no);
    for (; ktail && t == nk - 2; ++t) iteration(t, no, no, yes);
    for (; t < nk; ++t) iteration(t, no, no, no);
    full_epilogue(cur);
    } else {
    // ---- the direct-copy form on a persistent grid: each workgroup takes one tile of
    // each round of `grid` tiles until a round has none for it (K a multiple of 32
    // with more than D k-tiles, checked by the host), then, with stream-K, the pieces
    // of its share of the tail; a piece runs as a tile whose k-tiles are the piece's
    // (its sources start at the piece's first k, and it has at least D + 1 k-tiles).
    // Below, "tile" means such a unit. The stream of k-tile copies runs on across
    // tiles: the last D iterations of
    // a tile, which have no k-tile of their own left to copy, copy k-tiles 0 .. D-1 of
    // the workgroup's next tile into the stages that follow, so the next tile starts
    // with its first D k-tiles in LDS and no pipeline fill. The finished tile's
    // epilogue goes through the one stage the next tile does not yet occupy (that of
    // the finished tile's last k-tile), one 32 x 32 subtile (4 KB per wave) at a time.
    // Before its first global store each wave waits for all of its copies (only loads
    // are in flight then, and loads complete in order), so the next tile's first two
    // iterations need no memory wait and no later wait for a copy is counted across a
    // store issued after that copy: gfx950 counts stores and loads on one counter and
    // may complete them out of order.
    Src nxt;              // the next tile's sources
    uint32_t sb = 0;      // stage of the current tile's k-tile 0
    bool primed = false;  // k-tiles 0 .. D-1 of the current tile are complete in LDS
    for (;;) {
        Unit nu;
        const bool has_next = unit_at(round + 1, nu);
        if (has_next) make_src(nu, nxt);
        if (!primed) {
            for (int t = 0; t < D; ++t) {
#pragma unroll
                for (int i = 0; i < CPB; ++i) copy_a(cur, t, (uint32_t)t, i, no);
#pragma unroll
                for (int i = 0; i < CPB; ++i) copy_b(cur, t, (uint32_t)t, i, no);
            }
            vm_wait_n<2 * CPB * (D - 1)>();
            asm volatile("s_barrier" ::: "memory");
        }
#pragma unroll
        for (int r = 0; r < NREAD; ++r) read_one(f0, (int)(sb & 3u), 0, r);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        settle(f0);
        // One iteration (k-tile t, stage (sb + t) & 3). LAST: one of the last D, which
        // copies k-tile t + D - nk of the next tile (nk: this tile's k-tiles) when there is one (a uniform branch
        // around the copies) and otherwise nothing. A primed tile's first two
        // iterations skip the memory wait: their k-tiles 1 and 2 are complete.
        auto iteration = [&](int t, auto last_tag) {
            constexpr bool LAST = decltype(last_tag)::value;
            const uint32_t st = (sb + (uint32_t)t) & 3u;
            const uint32_t cst = (sb + (uint32_t)(t + D)) & 3u;
            const bool copy = !LAST || has_next;
            const Src& cs = LAST ? nxt : cur;
            const int ct = LAST ? t + D - cur.nk : t + D;
            step(f0, f1, (int)st, 1, copy, cs, ct, cst, 0, no);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (!(primed && t < 2)) {
                if (!LAST) vm_wait_n<2 * CPB * (D - 2) + CPB>();
                else vm_wait(copy ? 2 * CPB * (D - 2) + CPB : 2 * CPB * max(0, cur.nk - t - 2));
            }
            asm volatile("s_barrier" ::: "memory");
            settle(f1);
            step(f1, f0, (int)((st + 1) & 3u), 0, copy, cs, ct, cst, 1, no);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            settle(f0);
        };
        int t = 0;
        for (; t + D < cur.nk; ++t) iteration(t, no);
        for (; t < cur.nk; ++t) iteration(t, yes);
        // epilogue through the stage of this tile's last k-tile, (sb + nk - 1) & 3: 4 KB
        // per wave, one 32 x 32 subtile at a time (32 rows of 128 bytes, chunk c of row r
        // at c ^ (r & 7); the bank-conflict counter reads zero for both the
        // fragment-layout writes and the whole-row reads, where c ^ ((r >> 1) & 7) made
        // every write take two passes); each store instruction writes 8 rows of 128 bytes.
        // The row loop stays rolled, so that the store code (with a fused epilogue's
        // arithmetic) exists once per subtile.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
        __syncthreads();
        const uint32_t es = (sb + (uint32_t)(cur.nk - 1)) & 3u;
        char* slot = reinterpret_cast<char*>(wave < NW / 2 ? &sA[es][0] : &sB[es][0]) + (wave % (NW / 2)) * 4096;
        const int cm0 = cur.m0 + wrow0, cn0 = cur.n0 + wcol0;
        vm_wait_n<0>();  // the next tile's first k-tiles, before any store
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int c = rg * 2 + lh;
                    *reinterpret_cast<f32x4*>(slot + l32 * 128 + ((c ^ (l32 & 7)) << 4)) =
                        f32x4{acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
                }
                __builtin_amdgcn_wave_barrier();
#pragma clang loop unroll(disable)
                for (int it = 0; it < 4; ++it) {
                    const int row = it * 8 + (lane >> 3), c = lane & 7;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(slot + row * 128 + ((c ^ (row & 7)) << 4));
                    store4p(cur, cm0 + 32 * i + row, cn0 + 32 * j + c * 4, v);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (!has_next) break;
        // every wave's slot reads are done before the next tile refills this stage
        __syncthreads();
        primed = true;
        sb = (sb + (uint32_t)cur.nk) & 3u;
        cur = nxt;
        ++round;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < SJ; ++j) acc[i][j] = f32x16{};
    }
    }
}

// One tile per workgroup (grid x), or the persistent form. A split-K launch of the
// one-tile form (grid y = slices; not the persistent form) narrows A, B, K and C to
// the slice first: the slice's partial product goes to its workspace plane as plain
// fp32, and the fixed-order reduction applies any epilogue.
template <int DT, int OPB, int NW, bool REG, bool PERSIST = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void mfma32_sp(
    GemmArgs g) {
    if constexpr (!PERSIST) k_slice<2, OPB>(g);
    mfma32_sp_body<DT, OPB, NW, REG, PERSIST, false>(g, nullptr);
}

// Grouped calls on the persistent direct-copy form (8 waves; every problem 16-byte
// aligned with K a multiple of 32 and at least 128, row-major B with N a multiple of
// 8: checked by the host).
template <int DT, int OPB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma32_sp_grouped(GroupArgs ga) {
    GemmArgs g = {};
    g.xcd_remap = ga.xcd_remap;
    g.ep.kind = 0;
    mfma32_sp_body<DT, OPB, 8, false, true, true>(g, &ga);
}

}  // namespace dg
