// kernel_lds.h -- the LDS-staged SIMT kernel (fp32 FMAs from a register micro-tile).
#pragma once
#include "lds_layout.h"

namespace dg {

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
__device__ __forceinline__ void lds_tile(const GemmArgs& g, int tm, int tn) {
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
        vm_settled();  // nothing in flight here: the previous loads were stored
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
                const float* v = &acc[4 * q + r][4 * qb];
                store_run4(g, m, n, f32x4{v[0], v[1], v[2], v[3]});
            }
        }
}

template <int DT, int OPB, bool VEC, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void lds_gemm(GemmArgs g) {
    k_slice<(int)sizeof(typename Elem<DT>::type), OPB>(g);
    int tm, tn;
    tile_coords(g, tm, tn);
    lds_tile<DT, OPB, VEC, BM, BN, BK>(g, tm, tn);
}

// Persistent grouped form (see mfma16_gemm_grouped).
template <int DT, int OPB, bool VEC, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void lds_gemm_grouped(GroupArgs ga) {
    for (int t = persistent_id(ga.xcd_remap); t < ga.total_tiles; t += gridDim.x) {
        GemmArgs g;
        int tm, tn;
        group_tile<(int)sizeof(typename Elem<DT>::type)>(ga, t, g, tm, tn);
        __syncthreads();
        lds_tile<DT, OPB, VEC, BM, BN, BK>(g, tm, tn);
    }
}

}  // namespace dg
