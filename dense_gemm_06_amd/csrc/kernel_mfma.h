// kernel_mfma.h -- register-staged MFMA kernels (any shape, masked edges).
#pragma once
#include <type_traits>

#include "lds_layout.h"

namespace dg {

// MFMA kernels: operand roles.
//
// The matrix instruction computes D(16x16) += P(16 x k) * Q(k x 16) with D held
// as 4 consecutive rows of one column per lane (lane l: rows 4(l/16)..+3, column
// l%16). The kernels feed P = a 16 x k block of B^T (rows are n) and Q = a k x 16
// block of A^T (columns are m), so D = (A B)^T block and each lane ends up with
// 4 consecutive n of one row m of C: a 16-byte store per lane. P and Q use the
// same (lane, slot) -> k assignment, so the instruction's internal k order never
// matters: any k permutation applied identically to both operands leaves the sum
// unchanged.

// fp16 / bf16 inputs, v_mfma_f32_16x16x32: each lane supplies 8 consecutive k
// of one row of P and one column of Q (k = 8(l/16) + slot).
template <int DT, int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void mfma16_tile(const GemmArgs& g, int tm, int tn) {
    constexpr int NT = WM * WN * 64;
    constexpr int TWM = BM / WM, TWN = BN / WN;  // wave tile
    constexpr int SM = TWM / 16, SN = TWN / 16;  // 16 x 16 subtiles per wave
    constexpr int KC = BK / 8;                   // 16-byte chunks per k-row
    constexpr int NC = BN / 8;                   // 16-byte chunks per n-row
    constexpr int LA = BM * KC / NT;
    constexpr int LB = OPB == 0 ? BK * NC / NT : BN * KC / NT;
    static_assert(BK % 32 == 0 && KC == 8, "k tile must be 64 (8 chunks per row)");
    static_assert(LA >= 1 && LB >= 1 && (BM * KC) % NT == 0, "tile does not divide the thread count");
    static_assert(OPB == 1 || NC >= 8, "row-major B tile needs at least 8 chunks per row");

    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wmi = wave / WN, wni = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;
    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.B);

    // Global addresses: a wave-uniform base per k-tile plus a 32-bit per-thread
    // offset (the host bounds the leading dimensions so offsets fit).
    const uint16_t* __restrict__ Ablk = A + (size_t)m0 * g.lda;
    const uint16_t* __restrict__ Bblk = OPB == 0 ? B + n0 : B + (size_t)n0 * g.ldb;
    const uint32_t lda = (uint32_t)g.lda, ldb = (uint32_t)g.ldb;
    const int mlim = M - m0, nlim = N - n0;
    const bool interior = mlim >= BM && nlim >= BN;  // uniform: no row/column masking needed
    uint16_t ra[LA][8], rb[LB][8];
    auto load_tiles = [&](int kt) {
        const int k0 = kt * BK;
        const uint16_t* Ak = Ablk + k0;
        const uint16_t* Bk = OPB == 0 ? Bblk + (size_t)k0 * g.ldb : Bblk + k0;
        if (interior && k0 + BK <= K) {
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
                load_chunk_full<uint16_t, 8, VEC>(ra[p], Ak + (row * lda + c * 8));
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int idx = tid + NT * p;
                const int row = OPB == 0 ? idx / NC : idx / KC, c = OPB == 0 ? idx % NC : idx % KC;
                load_chunk_full<uint16_t, 8, VEC>(rb[p], Bk + (row * ldb + c * 8));
            }
            return;
        }
        vm_settled();  // nothing in flight here: the previous loads were stored
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
            const int valid = row < mlim ? min(8, K - k0 - c * 8) : 0;
            load_chunk<uint16_t, 8, VEC>(ra[p], Ak + (row * lda + c * 8), valid);
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + NT * p;
            if (OPB == 0) {
                const int row = idx / NC, c = idx % NC;
                const int valid = k0 + row < K ? min(8, nlim - c * 8) : 0;
                load_chunk<uint16_t, 8, VEC>(rb[p], Bk + (row * ldb + c * 8), valid);
            } else {
                const int row = idx / KC, c = idx % KC;
                const int valid = row < nlim ? min(8, K - k0 - c * 8) : 0;
                load_chunk<uint16_t, 8, VEC>(rb[p], Bk + (row * ldb + c * 8), valid);
            }
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
            *reinterpret_cast<u32x4*>(&sA[buf][row * BK + ((c ^ kmaj_swz(row)) << 3)]) =
                *reinterpret_cast<const u32x4*>(ra[p]);
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + NT * p;
            if (OPB == 0) {
                const int row = idx / NC, c = idx % NC;
                *reinterpret_cast<u32x4*>(&sB[buf][row * BN + ((c ^ nmaj_swz<NC>(row)) << 3)]) =
                    *reinterpret_cast<const u32x4*>(rb[p]);
            } else {
                const int row = idx / KC, c = idx % KC;
                *reinterpret_cast<u32x4*>(&sB[buf][row * BK + ((c ^ kmaj_swz(row)) << 3)]) =
                    *reinterpret_cast<const u32x4*>(rb[p]);
            }
        }
    };

    f32x4 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            u32x4 qa[SM], pb[SN];
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int r = wmi * TWM + i * 16 + l16;
                qa[i] = *reinterpret_cast<const u32x4*>(&sA[cur][r * BK + (((ks * 4 + lg) ^ kmaj_swz(r)) << 3)]);
            }
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                if (OPB == 0) {
                    // transpose reads: within each 16-lane group, lane i addresses row
                    // kb + i/4 at columns nb + 4(i%4); lane j receives column nb + j of
                    // rows kb..kb+3 (4 consecutive k).
                    const int nb = wni * TWN + j * 16;
                    const int col = nb + ((l16 & 3) << 2);
                    u32x2 h[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int krow = ks * 32 + lg * 8 + hh * 4 + (l16 >> 2);
                        const uint16_t* p =
                            &sB[cur][krow * BN + (((col >> 3) ^ nmaj_swz<NC>(krow)) << 3) + (col & 7)];
                        if (DT == DT_F16) {
                            fp16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4f16(DG_LDS_PTR(fp16x4_t, p));
                            h[hh] = __builtin_bit_cast(u32x2, t);
                        } else {
                            bf16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(DG_LDS_PTR(bf16x4_t, p));
                            h[hh] = __builtin_bit_cast(u32x2, t);
                        }
                    }
                    pb[j] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
                } else {
                    const int r = wni * TWN + j * 16 + l16;
                    pb[j] = *reinterpret_cast<const u32x4*>(&sB[cur][r * BK + (((ks * 4 + lg) ^ kmaj_swz(r)) << 3)]);
                }
            }
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    if (DT == DT_F16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(f16x8, pb[j]), __builtin_bit_cast(f16x8, qa[i]), acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, pb[j]), __builtin_bit_cast(bf16x8, qa[i]), acc[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < nk) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane owns C[m][n..n+3]
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int m = m0 + wmi * TWM + i * 16 + l16;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const int n = n0 + wni * TWN + j * 16 + lg * 4;
            store_run4(g, m, n, acc[i][j]);
        }
    }
}

template <int DT, int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, (BM / WM) * (BN / WN) >= 128 * 128 ? 1 : 8)))
void mfma16_gemm(GemmArgs g) {
    k_slice<2, OPB>(g);
    int tm, tn;
    tile_coords(g, tm, tn);
    mfma16_tile<DT, OPB, VEC, BM, BN, BK, WM, WN>(g, tm, tn);
}

// Persistent grouped form: each workgroup takes linear tiles id, id + grid, ...
// of all problems; the barrier before each tile keeps the previous tile's LDS
// reads ahead of the next tile's LDS writes.
template <int DT, int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, (BM / WM) * (BN / WN) >= 128 * 128 ? 1 : 8)))
void mfma16_gemm_grouped(GroupArgs ga) {
    for (int t = persistent_id(ga.xcd_remap); t < ga.total_tiles; t += gridDim.x) {
        GemmArgs g;
        int tm, tn;
        group_tile<2>(ga, t, g, tm, tn);
        __syncthreads();
        mfma16_tile<DT, OPB, VEC, BM, BN, BK, WM, WN>(g, tm, tn);
    }
}

// fp32 inputs, v_mfma_f32_16x16x4_f32: each lane supplies one k of one row of P
// and one column of Q per instruction. Four consecutive instructions (steps
// s = 0..3) take k = 4(l/16) + s, so a lane reads one float4 along k of A (and
// of a column-major B) and uses one component per step.
//
// Row-major B: a lane reads a float4 along n instead; P subtile u of a 64-wide
// group holds the columns n = 4(l%16) + u, so the four subtiles share one read
// and, at the store, a lane owns 16 consecutive n of one row of C.
//
// KG = 2 or 4 splits K inside the workgroup: KG groups of WM x WN waves, each with
// its own LDS stages, take k-tiles kg, kg + KG, ...; at the end groups 1 .. KG-1
// hand their accumulators to group 0 through LDS and group 0 adds them in group
// order (group 0's sum first, a fixed order) and stores. With one wave per SIMD a
// matrix instruction stream issues well below the unit's rate; the extra groups add
// waves per SIMD for tiles too small to hold more waves, and shorten each wave's
// chain of k-tiles where K is short.
//
// ST = 3 keeps three LDS stages instead of two, so that the fragments of the next
// k-tile can be read before the barrier that ends the current one: tile t + 1 was
// stored one iteration earlier, and the stage being filled (t + 2) is the one
// every wave finished reading before the previous barrier. Fragments are double-
// buffered by halves of the k-tile: each half's reads are issued while the other
// half's MFMAs run, so no MFMA waits on an LDS read that was issued just before it.
template <int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN, int KG = 1, int ST = 2>
__device__ __forceinline__ void mfma32_tile(const GemmArgs& g, int tm, int tn) {
    static_assert(KG == 1 || KG == 2 || KG == 4, "k groups");
    static_assert(ST == 2 || (ST == 3 && BK == 32), "three stages: k-tiles of 32");
    constexpr int NT = WM * WN * 64;  // threads of one k group
    constexpr int TWM = BM / WM, TWN = BN / WN;
    constexpr int SM = TWM / 16, SN = TWN / 16, QN = TWN / 64;
    constexpr int KC = BK / 4;  // 16-byte chunks per k-row
    constexpr int NC = BN / 4;  // 16-byte chunks per n-row
    constexpr int LA = BM * KC / NT;
    constexpr int LB = OPB == 0 ? BK * NC / NT : BN * KC / NT;
    static_assert(KC == 8, "k tile must be 32 (8 chunks per row)");
    static_assert(OPB == 1 || TWN % 64 == 0, "row-major B needs 64-wide wave tiles");
    static_assert(LA >= 1 && LB >= 1 && (BM * KC) % NT == 0, "tile does not divide the thread count");

    __shared__ __attribute__((aligned(16))) float sAg[KG][ST][BM * BK];
    __shared__ __attribute__((aligned(16))) float sBg[KG][ST][BN * BK];

    const int kg = KG == 1 ? 0 : (int)threadIdx.x / NT;  // uniform per wave
    float(&sA)[ST][BM * BK] = sAg[kg];
    float(&sB)[ST][BN * BK] = sBg[kg];
    const int tid = (int)threadIdx.x - kg * NT, lane = tid & 63, wave = tid >> 6;
    const int wmi = wave / WN, wni = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;
    const float* __restrict__ A = static_cast<const float*>(g.A);
    const float* __restrict__ B = static_cast<const float*>(g.B);

    const float* __restrict__ Ablk = A + (size_t)m0 * g.lda;
    const float* __restrict__ Bblk = OPB == 0 ? B + n0 : B + (size_t)n0 * g.ldb;
    const uint32_t lda = (uint32_t)g.lda, ldb = (uint32_t)g.ldb;
    const int mlim = M - m0, nlim = N - n0;
    const bool interior = mlim >= BM && nlim >= BN;  // uniform: no row/column masking needed
    float ra[LA][4], rb[LB][4];
    auto load_into = [&](float (&da)[LA][4], float (&db)[LB][4], int kt) {
        const int k0 = kt * BK;
        const float* Ak = Ablk + k0;
        const float* Bk = OPB == 0 ? Bblk + (size_t)k0 * g.ldb : Bblk + k0;
        if (interior && k0 + BK <= K) {
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
                load_chunk_full<float, 4, VEC>(da[p], Ak + (row * lda + c * 4));
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int idx = tid + NT * p;
                const int row = OPB == 0 ? idx / NC : idx / KC, c = OPB == 0 ? idx % NC : idx % KC;
                load_chunk_full<float, 4, VEC>(db[p], Bk + (row * ldb + c * 4));
            }
            return;
        }
        vm_settled();  // nothing in flight here: the previous loads were stored
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
            const int valid = row < mlim ? min(4, K - k0 - c * 4) : 0;
            load_chunk<float, 4, VEC>(da[p], Ak + (row * lda + c * 4), valid);
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + NT * p;
            if (OPB == 0) {
                const int row = idx / NC, c = idx % NC;
                const int valid = k0 + row < K ? min(4, nlim - c * 4) : 0;
                load_chunk<float, 4, VEC>(db[p], Bk + (row * ldb + c * 4), valid);
            } else {
                const int row = idx / KC, c = idx % KC;
                const int valid = row < nlim ? min(4, K - k0 - c * 4) : 0;
                load_chunk<float, 4, VEC>(db[p], Bk + (row * ldb + c * 4), valid);
            }
        }
    };
    auto load_tiles = [&](int kt) { load_into(ra, rb, kt); };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
            *reinterpret_cast<f32x4*>(&sA[buf][row * BK + ((c ^ kmaj_swz(row)) << 2)]) =
                f32x4{ra[p][0], ra[p][1], ra[p][2], ra[p][3]};
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + NT * p;
            if (OPB == 0) {
                const int row = idx / NC, c = idx % NC;
                *reinterpret_cast<f32x4*>(&sB[buf][row * BN + (c << 2)]) =
                    f32x4{rb[p][0], rb[p][1], rb[p][2], rb[p][3]};
            } else {
                const int row = idx / KC, c = idx % KC;
                *reinterpret_cast<f32x4*>(&sB[buf][row * BK + ((c ^ kmaj_swz(row)) << 2)]) =
                    f32x4{rb[p][0], rb[p][1], rb[p][2], rb[p][3]};
            }
        }
    };

    f32x4 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // group kg takes k-tiles kg, kg + KG, ...: nkg of them; every group runs the same
    // number of iterations (nl) so that all threads reach every barrier
    const int nk = (K + BK - 1) / BK;
    const int nkg = (nk - kg + KG - 1) / KG, nl = (nk + KG - 1) / KG;
    // k-tile of iteration lt for this group (at or past nk for a group with fewer
    // k-tiles than nl: the masked loads then bring zeros, which add nothing)
    auto ktile = [&](int lt) { return lt * KG + kg; };
    auto compute = [&](int cur) {
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            f32x4 qa[SM];
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int r = wmi * TWM + i * 16 + l16;
                qa[i] = *reinterpret_cast<const f32x4*>(&sA[cur][r * BK + ((((kk >> 2) + lg) ^ kmaj_swz(r)) << 2)]);
            }
            if (OPB == 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int krow = kk + 4 * lg + s;
                    f32x4 pq[QN];
#pragma unroll
                    for (int q = 0; q < QN; ++q)
                        pq[q] = *reinterpret_cast<const f32x4*>(&sB[cur][krow * BN + wni * TWN + q * 64 + 4 * l16]);
#pragma unroll
                    for (int i = 0; i < SM; ++i)
#pragma unroll
                        for (int q = 0; q < QN; ++q)
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                acc[i][4 * q + u] =
                                    __builtin_amdgcn_mfma_f32_16x16x4f32(pq[q][u], qa[i][s], acc[i][4 * q + u], 0, 0, 0);
                }
            } else {
                f32x4 pb[SN];
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const int r = wni * TWN + j * 16 + l16;
                    pb[j] = *reinterpret_cast<const f32x4*>(&sB[cur][r * BK + ((((kk >> 2) + lg) ^ kmaj_swz(r)) << 2)]);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < SM; ++i)
#pragma unroll
                        for (int j = 0; j < SN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pb[j][s], qa[i][s], acc[i][j], 0, 0, 0);
            }
        }
    };
    if constexpr (ST == 3) {
        // one half k-tile (16 k) of fragments: A as in compute(); B as four k-rows
        // (row-major) or SN column subtiles (column-major)
        struct Frag {
            f32x4 a[SM];
            f32x4 b[OPB == 0 ? 4 * QN : SN];
        };
        auto read_frag = [&](Frag& f, int buf, int kk) {
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int r = wmi * TWM + i * 16 + l16;
                f.a[i] = *reinterpret_cast<const f32x4*>(&sA[buf][r * BK + ((((kk >> 2) + lg) ^ kmaj_swz(r)) << 2)]);
            }
            if (OPB == 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int q = 0; q < QN; ++q)
                        f.b[s * QN + q] = *reinterpret_cast<const f32x4*>(
                            &sB[buf][(kk + 4 * lg + s) * BN + wni * TWN + q * 64 + 4 * l16]);
            } else {
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const int r = wni * TWN + j * 16 + l16;
                    f.b[j] = *reinterpret_cast<const f32x4*>(&sB[buf][r * BK + ((((kk >> 2) + lg) ^ kmaj_swz(r)) << 2)]);
                }
            }
        };
        // store chunk p (A's LA chunks, then B's LB) of the staged k-tile into stage buf
        auto store_chunk = [&](const float (&da)[LA][4], const float (&db)[LB][4], int buf, int p) {
            if (p < LA) {
                const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
                *reinterpret_cast<f32x4*>(&sA[buf][row * BK + ((c ^ kmaj_swz(row)) << 2)]) =
                    f32x4{da[p][0], da[p][1], da[p][2], da[p][3]};
            } else {
                const int q = p - LA, idx = tid + NT * q;
                if (OPB == 0) {
                    const int row = idx / NC, c = idx % NC;
                    *reinterpret_cast<f32x4*>(&sB[buf][row * BN + (c << 2)]) =
                        f32x4{db[q][0], db[q][1], db[q][2], db[q][3]};
                } else {
                    const int row = idx / KC, c = idx % KC;
                    *reinterpret_cast<f32x4*>(&sB[buf][row * BK + ((c ^ kmaj_swz(row)) << 2)]) =
                        f32x4{db[q][0], db[q][1], db[q][2], db[q][3]};
                }
            }
        };
        // the MFMAs of step s (one k of each lane's float4) of a half k-tile
        auto mma_step = [&](const Frag& f, int s) {
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                if (OPB == 0) {
#pragma unroll
                    for (int q = 0; q < QN; ++q)
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            acc[i][4 * q + u] =
                                __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[s * QN + q][u], f.a[i][s], acc[i][4 * q + u], 0, 0, 0);
                } else {
#pragma unroll
                    for (int j = 0; j < SN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[j][s], f.a[i][s], acc[i][j], 0, 0, 0);
                }
            }
        };
        auto mma = [&](const Frag& f) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    if (OPB == 0) {
#pragma unroll
                        for (int q = 0; q < QN; ++q)
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                acc[i][4 * q + u] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[s * QN + q][u], f.a[i][s],
                                                                                         acc[i][4 * q + u], 0, 0, 0);
                    } else {
#pragma unroll
                        for (int j = 0; j < SN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[j][s], f.a[i][s], acc[i][j], 0, 0, 0);
                    }
                }
        };
        Frag f0, f1;
        if (nl > 0) {
            load_tiles(ktile(0));
            store_tiles(0);
        }
        if (nl > 1) {
            load_tiles(ktile(1));
            store_tiles(1);
        }
        __syncthreads();
        if (nl > 0) read_frag(f0, 0, 0);
        // accumulators in the accumulation registers (measured 0.6% faster than in
        // the vector registers at 4096^3 and 8192^3)
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j) asm volatile("" : "+a"(acc[i][j]));
        int cur = 0;  // lt % 3
        for (int lt = 0; lt < nl; ++lt) {
            const int nxt = cur == 2 ? 0 : cur + 1, far = nxt == 2 ? 0 : nxt + 1;
            if (lt + 2 < nl) load_tiles(ktile(lt + 2));
            read_frag(f1, cur, 16);
            // the compiler would sink the reads below the MFMAs that should hide them
            __builtin_amdgcn_sched_barrier(0);
            mma(f0);
            __builtin_amdgcn_sched_barrier(0);
            // unconditional: after the last k-tile this reads a stage whose values go
            // unused, and a branch here would make the compiler wait for these reads
            // before the MFMAs below
            read_frag(f0, nxt, 0);
            __builtin_amdgcn_sched_barrier(0);
            // The LDS writes of tile t + 2 go between the MFMA steps of this half
            // rather than all at once before the barrier. Stage `far` is free for the
            // whole iteration; without a new tile (the last two iterations) the stale
            // registers land in a stage that is never read again.
            constexpr int NCH = LA + LB, PER = (NCH + 2) / 3;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                mma_step(f1, st);
                __builtin_amdgcn_sched_barrier(0);
                if (st < 3) {
#pragma unroll
                    for (int p = st * PER; p < NCH && p < (st + 1) * PER; ++p) store_chunk(ra, rb, far, p);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
            cur = nxt;
        }
    } else {
        if (nkg > 0) {
            load_tiles(kg);
            store_tiles(0);
        }
        __syncthreads();
        for (int lt = 0; lt < nl; ++lt) {
            const int cur = lt & 1;
            if (lt + 1 < nkg) load_tiles((lt + 1) * KG + kg);
            if (lt < nkg) compute(cur);
            if (lt + 1 < nkg) store_tiles(cur ^ 1);
            __syncthreads();
        }
    }
    if constexpr (KG > 1) {
        // the accumulators of groups 1 .. KG-1 through LDS (each group's own A stages,
        // free after the last barrier), lane-major so that consecutive lanes touch
        // consecutive words; group 0 adds them in group order
        static_assert(BM * BN <= ST * BM * BK, "reduction buffer");
        if (kg != 0) {
            float* red = &sAg[kg][0][0];
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[(((wave * SM + i) * SN + j) * 4 + e) * 64 + lane] = acc[i][j][e];
        }
        __syncthreads();
        if (kg != 0) return;
#pragma unroll
        for (int q = 1; q < KG; ++q) {
            const float* red = &sAg[q][0][0];
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] += red[(((wave * SM + i) * SN + j) * 4 + e) * 64 + lane];
        }
    }

#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int m = m0 + wmi * TWM + i * 16 + l16;
        if (m >= M) continue;
        if (OPB == 0) {
#pragma unroll
            for (int q = 0; q < QN; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = n0 + wni * TWN + q * 64 + 16 * lg + 4 * r;
                    store_run4(g, m, n,
                               f32x4{acc[i][4 * q][r], acc[i][4 * q + 1][r], acc[i][4 * q + 2][r], acc[i][4 * q + 3][r]});
                }
        } else {
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const int n = n0 + wni * TWN + j * 16 + lg * 4;
                store_run4(g, m, n, acc[i][j]);
            }
        }
    }
}

template <int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN, int KG = 1, int ST = 2>
__global__ __launch_bounds__(WM * WN * 64 * KG) void mfma32_gemm(GemmArgs g) {
    k_slice<4, OPB>(g);
    int tm, tn;
    tile_coords(g, tm, tn);
    mfma32_tile<OPB, VEC, BM, BN, BK, WM, WN, KG, ST>(g, tm, tn);
}

template <int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void mfma32_gemm_grouped(GroupArgs ga) {
    for (int t = persistent_id(ga.xcd_remap); t < ga.total_tiles; t += gridDim.x) {
        GemmArgs g;
        int tm, tn;
        group_tile<4>(ga, t, g, tm, tn);
        __syncthreads();
        mfma32_tile<OPB, VEC, BM, BN, BK, WM, WN>(g, tm, tn);
    }
}

}  // namespace dg
