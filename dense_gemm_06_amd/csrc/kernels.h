// kernels.h -- the GEMM kernels, C = A @ B with fp32 accumulation, for gfx950.
//
// Two kernel families, both built on the block tiling of "Shared memory and
// tensor cores" (section 13.3: a block stages a tile of A and of B in on-chip
// memory, waits at a barrier, reuses the tiles from there, and waits again
// before they are overwritten) and on the refinements listed in its section
// 13.10 (double buffering, 16-byte global loads, swizzled shared layouts, warp
// (wave) tiling):
//
//   lds_gemm    -- the LDS-staged SIMT kernel: each of 256 threads owns a
//                  register micro-tile (section 13.7) and does fp32 FMAs.
//   mfma16_gemm -- fp16/bf16 inputs on v_mfma_f32_16x16x32_{f16,bf16}, the
//                  CDNA4 counterpart of the chapter's 16x16x16 tensor-core
//                  operation (section 13.8: products exact, sums in fp32).
//   mfma32_gemm -- fp32 inputs on v_mfma_f32_16x16x4_f32 (full fp32 products
//                  and sums; gfx950 has no reduced-precision fp32 matrix op).
//
// Common structure: two LDS stages; the next k-tile is loaded from global memory
// into registers before the current one is consumed and written to the other
// stage afterwards, so one barrier per k-tile separates the write of a stage
// from its reads (read-after-write) and the reads of a stage from its next
// overwrite (write-after-read). Every thread of a workgroup reaches every
// barrier: edge handling is done by zero-filled loads and guarded stores, never
// by an early exit.
//
// Edges: loads of elements outside the matrix (row >= M or N, k >= K) return
// zero and are never dereferenced; stores outside C are skipped. The VEC
// template flag selects 16-byte global loads (requires 16-byte aligned bases
// and leading dimensions that are multiples of 16 bytes; the host checks) and
// otherwise element-wise loads.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace dg {

// ---------------------------------------------------------------------------
// LDS layouts
//
// gfx950 LDS, as measured with bank-conflict counters on this hardware: 64 banks
// of 4 bytes (a 256-byte period). 8-byte reads, including the transpose reads,
// are served 32 consecutive lanes at a time. 16-byte reads are served in four
// phases of 16 lanes built from lane quads: lane l is in phase
// (l / 32, parity of bits 2..4 of l), e.g. lanes 0-3, 12-15, 20-23, 24-27.
// A phase is conflict-free when its lanes touch distinct 16-byte positions of
// the 256-byte bank period (section 13.6's rule, with these banks and phases).
//
// K-major tiles (A, and B when it is column-major): row r holds BK consecutive k
// as 16-byte chunks (128-byte rows); chunk c is stored at position c ^ (r & 7).
// A fragment read takes rows r0..r0+15 at chunk columns c0 (lanes 0-15) and
// c0+1 (lanes 16-31); under the phase grouping above every phase then covers all
// 16 positions once. No padding, and 16-byte accesses stay aligned.
__device__ __forceinline__ int kmaj_swz(int r) { return r & 7; }

// N-major tile of a 16-bit row-major B: row k holds BN consecutive n as 16-byte
// chunks; chunk c is stored at c ^ nmaj_swz(k). The transpose reads of one
// 32-lane phase touch 8 rows {8g + 4h + r : g in 0..1, r in 0..3} at two
// neighbouring chunks; the eight even XOR values 2((k & 3) | 4((k >> 3) & 1))
// send the even chunk to the 8 even positions and the odd chunk to the 8 odd
// ones, so the phase hits all 16 positions once.
template <int CHUNKS>
__device__ __forceinline__ int nmaj_swz(int k) {
    return (((k & 3) | (((k >> 3) & 1) << 2)) << 1) & (CHUNKS - 1);
}

// ---------------------------------------------------------------------------
// LDS-staged SIMT kernel.
//
// 256 threads as 16 x 16; thread (ty, tx) owns rows q*64 + 4ty + {0..3} and
// columns q*64 + 4tx + {0..3} of the block tile (q < BM/64, BN/64), so its loads
// from LDS are 16-byte vectors and neighbouring lanes touch neighbouring words
// (the coalesced upcast layout of "GPU architecture and mapping kernels", 12.8).
// A is stored transposed in LDS (k rows, m contiguous) and B with k rows, both
// converted to fp32, with an XOR swizzle at float4 granularity on the transposed
// stores.
template <int DT, int OPB, bool VEC, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void lds_gemm(GemmArgs g) {
    typedef typename Elem<DT>::type T;
    constexpr int V = Elem<DT>::vec;   // elements per 16-byte chunk
    constexpr int RA = BM / 64, RB = BN / 64;
    constexpr int TM = 4 * RA, TN = 4 * RB;
    constexpr int CA = BK / V;         // chunks per k-contiguous row
    constexpr int LA = BM * CA / 256;  // A chunks per thread
    constexpr int CBN = BN / V;        // chunks per n-contiguous row of B
    constexpr int LB = OPB == 0 ? BK * CBN / 256 : BN * CA / 256;
    static_assert(LA >= 1 && LB >= 1 && (BM * CA) % 256 == 0, "tile does not divide the thread count");
    static_assert(BK / V <= 4, "transposed-store swizzle assumes at most 4 chunks per row");

    __shared__ __attribute__((aligned(16))) float sA[2][BK * BM];
    __shared__ __attribute__((aligned(16))) float sB[2][BK * BN];

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;
    const T* __restrict__ A = static_cast<const T*>(g.A);
    const T* __restrict__ B = static_cast<const T*>(g.B);

    // quad swizzle of the transposed stores: 2 * ((k / V) mod 4)
    auto tsw = [](int k) { return ((k / V) & 3) << 1; };

    const T* __restrict__ Ablk = A + (size_t)m0 * g.lda;
    const T* __restrict__ Bblk = OPB == 0 ? B + n0 : B + (size_t)n0 * g.ldb;
    const uint32_t lda = (uint32_t)g.lda, ldb = (uint32_t)g.ldb;
    const int mlim = M - m0, nlim = N - n0;
    const bool interior = mlim >= BM && nlim >= BN;  // uniform: no row/column masking needed
    T ra[LA][V], rb[LB][V];
    auto load_tiles = [&](int kt) {
        const int k0 = kt * BK;
        const T* Ak = Ablk + k0;
        const T* Bk = OPB == 0 ? Bblk + (size_t)k0 * g.ldb : Bblk + k0;
        if (interior && k0 + BK <= K) {
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int idx = tid + 256 * p, row = idx / CA, c = idx % CA;
                load_chunk_full<T, V, VEC>(ra[p], Ak + (row * lda + c * V));
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int idx = tid + 256 * p;
                const int row = OPB == 0 ? idx / CBN : idx / CA, c = OPB == 0 ? idx % CBN : idx % CA;
                load_chunk_full<T, V, VEC>(rb[p], Bk + (row * ldb + c * V));
            }
            return;
        }
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + 256 * p, row = idx / CA, c = idx % CA;
            const int valid = row < mlim ? min(V, K - k0 - c * V) : 0;
            load_chunk<T, V, VEC>(ra[p], Ak + (row * lda + c * V), valid);
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + 256 * p;
            if (OPB == 0) {
                const int row = idx / CBN, c = idx % CBN;
                const int valid = k0 + row < K ? min(V, nlim - c * V) : 0;
                load_chunk<T, V, VEC>(rb[p], Bk + (row * ldb + c * V), valid);
            } else {
                const int row = idx / CA, c = idx % CA;
                const int valid = row < nlim ? min(V, K - k0 - c * V) : 0;
                load_chunk<T, V, VEC>(rb[p], Bk + (row * ldb + c * V), valid);
            }
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + 256 * p, row = idx / CA, c = idx % CA;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int k = c * V + e;
                sA[buf][k * BM + (((row >> 2) ^ tsw(k)) << 2) + (row & 3)] = decode<DT>(ra[p][e]);
            }
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + 256 * p;
            if (OPB == 0) {
                const int row = idx / CBN, c = idx % CBN;
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    f32x4 v = {decode<DT>(rb[p][4 * q]), decode<DT>(rb[p][4 * q + 1]),
                               decode<DT>(rb[p][4 * q + 2]), decode<DT>(rb[p][4 * q + 3])};
                    *reinterpret_cast<f32x4*>(&sB[buf][row * BN + (c * V / 4 + q) * 4]) = v;
                }
            } else {
                const int row = idx / CA, c = idx % CA;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const int k = c * V + e;
                    sB[buf][k * BN + (((row >> 2) ^ tsw(k)) << 2) + (row & 3)] = decode<DT>(rb[p][e]);
                }
            }
        }
    };

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll 2
        for (int kk = 0; kk < BK; ++kk) {
            float a[TM], b[TN];
            const int bsw = OPB == 0 ? 0 : tsw(kk);
#pragma unroll
            for (int q = 0; q < RA; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&sA[cur][kk * BM + (((q * 16 + ty) ^ tsw(kk)) << 2)]);
                a[4 * q] = v[0]; a[4 * q + 1] = v[1]; a[4 * q + 2] = v[2]; a[4 * q + 3] = v[3];
            }
#pragma unroll
            for (int q = 0; q < RB; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&sB[cur][kk * BN + (((q * 16 + tx) ^ bsw) << 2)]);
                b[4 * q] = v[0]; b[4 * q + 1] = v[1]; b[4 * q + 2] = v[2]; b[4 * q + 3] = v[3];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) store_tiles(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int q = 0; q < RA; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + q * 64 + ty * 4 + r;
            if (m >= M) continue;
#pragma unroll
            for (int qb = 0; qb < RB; ++qb) {
                const int n = n0 + qb * 64 + tx * 4;
                float* cp = g.C + (size_t)m * g.ldc + n;
                const float* v = &acc[4 * q + r][4 * qb];
                if (n + 3 < N && (reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                    *reinterpret_cast<f32x4*>(cp) = f32x4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) cp[e] = v[e];
                }
            }
        }
}

// ---------------------------------------------------------------------------
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
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, (BM / WM) * (BN / WN) >= 128 * 128 ? 1 : 8)))
void mfma16_gemm(GemmArgs g) {
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
    int tm, tn;
    tile_coords(g, tm, tn);
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
            float* cp = g.C + (size_t)m * g.ldc + n;
            const f32x4 v = acc[i][j];
            if (n + 3 < N && (reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                *reinterpret_cast<f32x4*>(cp) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) cp[e] = v[e];
            }
        }
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
template <int OPB, bool VEC, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void mfma32_gemm(GemmArgs g) {
    constexpr int NT = WM * WN * 64;
    constexpr int TWM = BM / WM, TWN = BN / WN;
    constexpr int SM = TWM / 16, SN = TWN / 16, QN = TWN / 64;
    constexpr int KC = BK / 4;  // 16-byte chunks per k-row
    constexpr int NC = BN / 4;  // 16-byte chunks per n-row
    constexpr int LA = BM * KC / NT;
    constexpr int LB = OPB == 0 ? BK * NC / NT : BN * KC / NT;
    static_assert(KC == 8, "k tile must be 32 (8 chunks per row)");
    static_assert(OPB == 1 || TWN % 64 == 0, "row-major B needs 64-wide wave tiles");
    static_assert(LA >= 1 && LB >= 1 && (BM * KC) % NT == 0, "tile does not divide the thread count");

    __shared__ __attribute__((aligned(16))) float sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) float sB[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wmi = wave / WN, wni = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
    int tm, tn;
    tile_coords(g, tm, tn);
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
    auto load_tiles = [&](int kt) {
        const int k0 = kt * BK;
        const float* Ak = Ablk + k0;
        const float* Bk = OPB == 0 ? Bblk + (size_t)k0 * g.ldb : Bblk + k0;
        if (interior && k0 + BK <= K) {
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
                load_chunk_full<float, 4, VEC>(ra[p], Ak + (row * lda + c * 4));
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int idx = tid + NT * p;
                const int row = OPB == 0 ? idx / NC : idx / KC, c = OPB == 0 ? idx % NC : idx % KC;
                load_chunk_full<float, 4, VEC>(rb[p], Bk + (row * ldb + c * 4));
            }
            return;
        }
#pragma unroll
        for (int p = 0; p < LA; ++p) {
            const int idx = tid + NT * p, row = idx / KC, c = idx % KC;
            const int valid = row < mlim ? min(4, K - k0 - c * 4) : 0;
            load_chunk<float, 4, VEC>(ra[p], Ak + (row * lda + c * 4), valid);
        }
#pragma unroll
        for (int p = 0; p < LB; ++p) {
            const int idx = tid + NT * p;
            if (OPB == 0) {
                const int row = idx / NC, c = idx % NC;
                const int valid = k0 + row < K ? min(4, nlim - c * 4) : 0;
                load_chunk<float, 4, VEC>(rb[p], Bk + (row * ldb + c * 4), valid);
            } else {
                const int row = idx / KC, c = idx % KC;
                const int valid = row < nlim ? min(4, K - k0 - c * 4) : 0;
                load_chunk<float, 4, VEC>(rb[p], Bk + (row * ldb + c * 4), valid);
            }
        }
    };
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
        if (kt + 1 < nk) store_tiles(cur ^ 1);
        __syncthreads();
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
                    float* cp = g.C + (size_t)m * g.ldc + n;
                    const f32x4 v = {acc[i][4 * q][r], acc[i][4 * q + 1][r], acc[i][4 * q + 2][r], acc[i][4 * q + 3][r]};
                    if (n + 3 < N && (reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                        *reinterpret_cast<f32x4*>(cp) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) cp[e] = v[e];
                    }
                }
        } else {
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const int n = n0 + wni * TWN + j * 16 + lg * 4;
                float* cp = g.C + (size_t)m * g.ldc + n;
                const f32x4 v = acc[i][j];
                if (n + 3 < N && (reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                    *reinterpret_cast<f32x4*>(cp) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) cp[e] = v[e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Ping-pong MFMA kernel for 16-bit inputs on full 256 x 256 tiles (M and N
// multiples of 256, K a multiple of 32, 16-byte aligned operands).
//
// The register-staged kernel above runs every wave through the same sequence
// (load, wait, MFMA, store, barrier), so the matrix unit idles whenever all
// waves wait on memory together. Here the 8 waves form two groups of 4, one
// wave of each group per SIMD, and the groups run one phase apart: in every
// phase one group issues a block of 32 MFMAs (16x16x32) from registers while the
// other reads its fragments of the next k-tile from LDS and starts direct
// global -> LDS copies (global_load_lds_dwordx4, no registers involved) three
// k-tiles ahead. One barrier ends each phase.
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
// 64-byte k-major rows: chunk c of row r is stored at c ^ ((r >> 1) & 3), which
// keeps the 16-byte fragment reads (16 rows x 4 chunks) conflict-free under the
// gfx950 phase rule above; the row-major B tile uses nmaj_swz like the
// register-staged kernel.
__device__ __forceinline__ int kmaj64_swz(int r) { return (r >> 1) & 3; }

// Swizzles for the 32x32x16 fragment reads of mfma16_dma (64-byte k-major rows read
// 32 rows at a time; 512-byte n-major rows read as 4 rows x 64 bytes per 32-lane
// transpose phase), conflict-free under the gfx950 rules above.
__device__ __forceinline__ int kmaj32_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int nmaj32_swz(int k) { return (k & 3) << 2; }

#define DG_GLB(p) ((__attribute__((address_space(1))) void*)(p))
#define DG_LDSV(p) ((__attribute__((address_space(3))) void*)(p))

template <int DT, int OPB>
__global__ __launch_bounds__(512) void mfma16_pp(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BK = 32, S = 4;
    constexpr int SA = BM * BK, SB = BN * BK;  // halfs per stage
    __shared__ __attribute__((aligned(1024))) uint16_t sA[S][SA];
    __shared__ __attribute__((aligned(1024))) uint16_t sB[S][SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, wl = wave & 3;
    const int l16 = lane & 15, lg = lane >> 4;
    int tm, tn;
    tile_coords(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = g.K / BK;
    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.B);

    // Direct copies: each wave issues 4 copies of 1 KB (64 lanes x 16 B) per tile.
    // Lane L of block b lands at LDS byte b*1024 + 16L, i.e. at a fixed swizzled
    // position; it loads the logical chunk that belongs there.
    const uint16_t* src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = wl * 4 + i;
        if (grp == 0 || OPB == 1) {
            const int row = b * 16 + (lane >> 2);
            const int c = (lane & 3) ^ kmaj64_swz(row);
            src[i] = grp == 0 ? A + (size_t)(m0 + row) * g.lda + c * 8 : B + (size_t)(n0 + row) * g.ldb + c * 8;
        } else {
            const int row = b * 2 + (lane >> 5);
            const int c = (lane & 31) ^ nmaj_swz<BN / 8>(row);
            src[i] = B + (size_t)row * g.ldb + n0 + c * 8;
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

    // qa: Q fragments (A rows); pb: P fragments of column-major B; ph: the two
    // 4-k halves of a row-major-B P fragment, read by transpose reads issued as
    // inline asm. The compiler cannot tell those reads from the in-flight LDS-DMA
    // writes and would otherwise wait for every copy (vmcnt(0)) before them; the
    // asm form leaves the ordering to the explicit waits of sync_phase. Their
    // results are combined into MFMA operands only after the lgkmcnt(0) wait and
    // barrier that end the phase.
    u32x4 qa[8], pb[4];
    u32x2 ph[4][2];
    auto load_frags = [&](int t) {
        const uint16_t* a = sA[t & 3];
        const uint16_t* bb = sB[t & 3];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = grp * 128 + i * 16 + l16;
            qa[i] = *reinterpret_cast<const u32x4*>(a + r * BK + ((lg ^ kmaj64_swz(r)) << 3));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (OPB == 0) {
                // transpose reads: in each 16-lane group, lane i addresses row kb + i/4 at
                // columns nb + 4(i%4); lane i then holds column nb + i of rows kb..kb+3.
                const int col = wl * 64 + j * 16 + ((l16 & 3) << 2);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int krow = lg * 8 + hh * 4 + (l16 >> 2);
                    const uint16_t* p = bb + krow * BN + (((col >> 3) ^ nmaj_swz<BN / 8>(krow)) << 3) + (col & 7);
                    const uint32_t addr = (uint32_t)reinterpret_cast<uintptr_t>(DG_LDSV(p));
                    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(ph[j][hh]) : "v"(addr));
                }
            } else {
                const int r = wl * 64 + j * 16 + l16;
                pb[j] = *reinterpret_cast<const u32x4*>(bb + r * BK + ((lg ^ kmaj64_swz(r)) << 3));
            }
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&]() {
        if (OPB == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) pb[j] = u32x4{ph[j][0][0], ph[j][0][1], ph[j][1][0], ph[j][1][1]};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (DT == DT_F16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, pb[j]),
                                                                      __builtin_bit_cast(f16x8, qa[i]), acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pb[j]),
                                                                       __builtin_bit_cast(bf16x8, qa[i]), acc[i][j], 0, 0, 0);
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

    // epilogue: lane owns C[m][n..n+3]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = m0 + grp * 128 + i * 16 + l16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wl * 64 + j * 16 + lg * 4;
            float* cp = g.C + (size_t)m * g.ldc + n;
            const f32x4 v = acc[i][j];
            if ((reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                *reinterpret_cast<f32x4*>(cp) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) cp[e] = v[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
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
                float* cp = g.C + (size_t)m * g.ldc + n;
                const f32x4 v = {acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
                if ((reinterpret_cast<uintptr_t>(cp) & 15) == 0) {
                    *reinterpret_cast<f32x4*>(cp) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) cp[e] = v[e];
                }
            }
    }
}

}  // namespace dg
