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

// Eight consecutive 16-bit elements from a 2-byte aligned address p, reading only
// those 16 bytes, as four 32-bit words: a chunk that starts 4-byte aligned is four
// aligned words; one that starts 2 bytes off is elements 1..6 as three aligned words
// plus elements 0 and 7 as halves. The three middle words are one load instruction
// for both kinds of lane (only the address differs), so a wave whose lanes mix the
// two alignments (rows of odd length) issues six loads where element-wise loading
// issues eight. (In the GEMM kernels' own loaders this measured slower than
// element-wise loads on the ragged 3001 x 5003 x 1037 problem, 130 us against 112.)
__device__ __forceinline__ u32x4 load8_u16(const uint16_t* p) {
    const bool odd = (reinterpret_cast<uintptr_t>(p) & 2) != 0;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p + (odd ? 1 : 2));  // 4-byte aligned either way
    const uint32_t m0 = q[0], m1 = q[1], m2 = q[2];  // elements 2..7 (aligned) or 1..6 (odd)
    uint32_t first, last = 0;
    if (odd) {
        first = p[0];
        last = p[7];
    } else {
        first = *reinterpret_cast<const uint32_t*>(p);  // elements 0, 1
    }
    if (!odd) return u32x4{first, m0, m1, m2};
    return u32x4{first | (m0 << 16), (m0 >> 16) | (m1 << 16), (m1 >> 16) | (m2 << 16), (m2 >> 16) | (last << 16)};
}

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
            w = load8_u16(reinterpret_cast<const uint16_t*>(src + r * ld + c0));
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
