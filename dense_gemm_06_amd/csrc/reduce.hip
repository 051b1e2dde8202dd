// reduce.hip -- the fixed-order reduction that completes a split-K product.
//
// Each K slice of a split launch wrote its partial product of C into its own
// plane of the caller's workspace; this kernel adds the planes in slice order
// 0, 1, ..., S-1 and writes C once, so the result does not depend on the order
// in which the slices ran (no atomics).
#include <algorithm>

#include "device_common.h"
#include "launch.h"

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
        for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(w + (size_t)s * (size_t)slice);
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

int launch_splitk_reduce(const float* work, int S, int64_t slice, int64_t work_ld, int M, int N, void* C,
                         int64_t ldc, const Epilogue& ep, hipStream_t stream) {
    const int64_t total = (int64_t)M * ((N + 3) / 4);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 4096));
    return launch_status(splitk_reduce, dim3(grid), dim3(256), stream, work, S, slice, work_ld, M, N, C, ldc, ep);
}

}  // namespace dg
