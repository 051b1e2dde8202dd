// reduce.hip -- the fixed-order reductions that complete a split-K or a stream-K
// product.
//
// Each K slice of a split launch wrote its partial product of C into its own
// plane of the caller's workspace; splitk_reduce adds the planes in slice order
// 0, 1, ..., S-1 and writes C once, so the result does not depend on the order
// in which the slices ran (no atomics). streamk_fixup does the same for the tail
// tiles of a stream-K launch whose k-tiles several workgroups shared: it adds each
// such tile's partial sums in k order.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "streamk.h"

namespace dg {

// One thread per 4 consecutive columns of a row, grid-stride. work_ld is a
// multiple of 4 and the workspace is 16-byte aligned, so every workspace read is
// one aligned 16-byte load; columns N..work_ld-1 of a plane are read (never
// written by the slices) but not stored.
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ work, int S, int64_t slice,
                                                     int64_t work_ld, int M, int N, void* __restrict__ Cv,
                                                     int64_t ldc, Epilogue ep) {
    const int quads = (N + 3) >> 2;
    const int64_t total = (int64_t)M * quads;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int i = (int)(q / quads);
        const int j = (int)(q - (int64_t)i * quads) * 4;
        const float* w = work + (size_t)i * (size_t)work_ld + j;
        f32x4 acc = *reinterpret_cast<const f32x4*>(w);
        // planes 1 .. S-1 in order, their loads issued four at a time (a load per
        // iteration would wait out one memory latency per plane)
        int s = 1;
        for (; s + 4 <= S; s += 4) {
            f32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4*>(w + (size_t)(s + u) * (size_t)slice);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += v[u];
        }
        for (; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(w + (size_t)s * (size_t)slice);
        if (ep.kind != 0) {
            // the fused epilogue applies to the complete sum
            for (int e = 0; e < 4; ++e)
                if (j + e < N)
                    store_out(Cv, ep.out_dt, (size_t)i * (size_t)ldc + j + e,
                              epilogue_value(ep, acc[e], (size_t)i * (size_t)ep.ldr + j + e, j + e));
            continue;
        }
        float* c = static_cast<float*>(Cv) + (size_t)i * (size_t)ldc + j;
        if (j + 4 <= N) {
            __builtin_memcpy(c, &acc, 16);  // one 16-byte store, at any element-aligned address
        } else {
            for (int e = 0; e < 4; ++e)
                if (j + e < N) c[e] = acc[e];
        }
    }
}

// Stream-K fixup: block (t, y) completes rows 16y .. 16y + 15 of tail tile t (tile
// tile0 + t of the linear order, placed by the same raster as the product kernel),
// if more than one workgroup shared its k-tiles; G is the number of workgroups the
// tail was dealt to. Each thread owns 4 runs of 4 columns (rows 16y + r + 4u). The
// partial sums (slot 2w + p of workgroup w's piece p, 256 x 256 fp32) are added in k
// order, i.e. in increasing w, the first one taken as it is; they are gathered four
// pieces at a time, so that a thread has up to sixteen loads in flight. (Grids of 32
// and 64 blocks per tile, with fewer runs per thread, measured slower: each block
// first works out the tile's pieces, which costs more than the loads it saves.)
__global__ __launch_bounds__(256) void streamk_fixup(const float* __restrict__ work, int G, int S, int KT, int tile0,
                                                     int tiles_m, int tiles_n, int group_m, int M, int N,
                                                     void* __restrict__ Cv, int64_t ldc, Epilogue ep) {
    const int t = blockIdx.x;
    const int64_t iters = (int64_t)S * KT, lo = (int64_t)t * KT, hi = lo + KT;
    const int w0 = sk_owner(lo, G, iters, KT);
    int64_t b0 = sk_bound(w0, G, iters, KT), b1 = sk_bound(w0 + 1, G, iters, KT);
    if (b1 >= hi) return;  // one piece: its workgroup stored C
    int tm, tn;
    raster(tile0 + t, tiles_m, tiles_n, group_m, tm, tn);
    const int r0 = blockIdx.y * 16 + (threadIdx.x >> 6), c = (threadIdx.x & 63) * 4;  // rows r0 + 4u
    f32x4 acc[4];
    bool first = true;
    int w = w0;
    for (;;) {
        // the next (up to) four pieces in the tile, in k order; b0, b1 bound share w
        const float* slot[4];
        int n = 0;
        while (n < 4 && w < G && b0 < hi) {
            if (b1 > b0 && b1 > lo) slot[n++] = work + (size_t)(2 * w + (b0 >= lo ? 0 : 1)) * 65536u;
            ++w;
            b0 = b1;
            if (w < G) b1 = sk_bound(w + 1, G, iters, KT);
        }
        if (n == 0) break;
        f32x4 v[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < n)
#pragma unroll
                for (int u = 0; u < 4; ++u) v[i][u] = *reinterpret_cast<const f32x4*>(slot[i] + (r0 + 4 * u) * 256 + c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < n)
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[u] = first && i == 0 ? v[i][u] : acc[u] + v[i][u];
        first = false;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tm * 256 + r0 + 4 * u, j = tn * 256 + c;
        if (i >= M || j >= N) continue;
        if (ep.kind != 0) {
            epilogue_run4_body(ep, Cv, ldc, N, i, j, acc[u]);
            continue;
        }
        float* cp = static_cast<float*>(Cv) + (size_t)i * (size_t)ldc + j;
        if (j + 4 <= N) {
            __builtin_memcpy(cp, &acc[u], 16);
        } else {
            for (int e = 0; e < 4; ++e)
                if (j + e < N) cp[e] = acc[u][e];
        }
    }
}

int launch_streamk_fixup(const float* work, int G, int S, int KT, int tile0, int tiles_m, int tiles_n, int group_m,
                         int M, int N, void* C, int64_t ldc, const Epilogue& ep, hipStream_t stream) {
    return launch_status(streamk_fixup, dim3((unsigned)S, 16), dim3(256), stream, work, G, S, KT, tile0, tiles_m,
                         tiles_n, group_m, M, N, C, ldc, ep);
}

int launch_splitk_reduce(const float* work, int S, int64_t slice, int64_t work_ld, int M, int N, void* C,
                         int64_t ldc, const Epilogue& ep, hipStream_t stream) {
    const int64_t total = (int64_t)M * ((N + 3) / 4);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 4096));
    return launch_status(splitk_reduce, dim3(grid), dim3(256), stream, work, S, slice, work_ld, M, N, C, ldc, ep);
}

}  // namespace dg
