// pack.hip -- copy the operands into zero-padded, 16-byte aligned buffers.
//
// Operands whose rows are not 16-byte aligned (or whose shapes are not whole
// tiles) can be copied once into a caller-provided workspace: rows padded to
// cols_p elements (a multiple of 16 bytes) and the matrix padded with zero rows
// and columns to rows_p x cols_p. The product then runs on aligned, whole-tile
// data; the zero padding adds exact zeros to every sum.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace dg {

// One thread per 16-byte chunk of a destination, grid-stride over the chunks of
// both destinations (A's first, then B's). Source elements outside rows x cols
// are never read.
template <typename T>
__global__ __launch_bounds__(256) void pack_pad(PackJob a, PackJob b, int64_t chunks_a, int64_t chunks_total) {
    constexpr int V = 16 / (int)sizeof(T);
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < chunks_total; q += (int64_t)gridDim.x * 256) {
        const bool first = q < chunks_a;
        const int64_t local = first ? q : q - chunks_a;
        const T* src = static_cast<const T*>(first ? a.src : b.src);
        T* dst = static_cast<T*>(first ? a.dst : b.dst);
        const int64_t ld = first ? a.ld : b.ld;
        const int rows = first ? a.rows : b.rows, cols = first ? a.cols : b.cols;
        const int64_t cols_p = first ? a.cols_p : b.cols_p;
        const int64_t per_row = cols_p / V;
        const int64_t r = local / per_row;
        const int c0 = (int)(local - r * per_row) * V;
        u32x4 w;
        if (sizeof(T) == 2 && r < rows && c0 + V <= cols) {
            // a whole chunk of 8 16-bit elements inside the source: 4-byte loads (16-bit
            // elements start on 2-byte boundaries, so a chunk is 4-byte aligned or 2 off)
            const uint16_t* p = reinterpret_cast<const uint16_t*>(src + r * ld + c0);
            if ((reinterpret_cast<uintptr_t>(p) & 3) == 0) {
                const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
                w = u32x4{q[0], q[1], q[2], q[3]};
            } else {
                // elements 1..6 as three aligned words, 0 and 7 on their own: nothing
                // outside the chunk is read
                const uint32_t* q = reinterpret_cast<const uint32_t*>(p + 1);
                const uint32_t d0 = q[0], d1 = q[1], d2 = q[2];
                const uint32_t e0 = p[0], e7 = p[7];
                w = u32x4{e0 | (d0 << 16), (d0 >> 16) | (d1 << 16), (d1 >> 16) | (d2 << 16), (d2 >> 16) | (e7 << 16)};
            }
        } else {
            T v[V];
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = (r < rows && c0 + e < cols) ? src[r * ld + c0 + e] : T(0);
            w = *reinterpret_cast<const u32x4*>(v);
        }
        *reinterpret_cast<u32x4*>(dst + r * cols_p + c0) = w;
    }
}

int launch_pack(int elem_size, const PackJob& a, const PackJob& b, hipStream_t stream) {
    const int V = 16 / elem_size;
    const int64_t chunks_a = (int64_t)a.rows_p * a.cols_p / V;
    const int64_t total = chunks_a + (int64_t)b.rows_p * b.cols_p / V;
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 8192));
    if (elem_size == 2)
        hipLaunchKernelGGL(pack_pad<uint16_t>, dim3(grid), dim3(256), 0, stream, a, b, chunks_a, total);
    else
        hipLaunchKernelGGL(pack_pad<float>, dim3(grid), dim3(256), 0, stream, a, b, chunks_a, total);
    return 0;
}

}  // namespace dg
