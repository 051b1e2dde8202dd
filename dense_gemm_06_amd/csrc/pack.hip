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

// Row of chunk n for rows of d chunks: the quotient n / d from a double-precision
// estimate, corrected by one step. For n < 2^51 the estimate is within one of the
// quotient. A 64-bit integer division is a long instruction sequence on this GPU.
// On the 3001 x 5003 x 1037 bf16 operands the whole packed call measured 1.5-2.5 us
// faster with this in one alternated session; a kernel trace of the copy alone shows
// the same 9.8 us average (minimum 8.7 against 9.3 us).
__device__ __forceinline__ int64_t chunk_row(int64_t n, int64_t d, double inv_d) {
    int64_t q = (int64_t)((double)n * inv_d);
    const int64_t r = n - q * d;
    if (r < 0) q -= 1;
    else if (r >= d) q += 1;
    return q;
}

// One thread per 16-byte chunk of a destination, grid-stride over the chunks of
// both destinations (A's first, then B's). Source elements outside rows x cols
// are never read. (Two, four or eight chunks per thread, 256 chunks apart, all
// loads before the stores, measured no faster on the 3001 x 5003 x 1037 bf16
// operands.)
template <typename T>
__global__ __launch_bounds__(256) void pack_pad(PackJob a, PackJob b, int64_t chunks_a, int64_t chunks_total) {
    constexpr int V = 16 / (int)sizeof(T);
    const double inv_a = 1.0 / (double)(a.cols_p / V), inv_b = 1.0 / (double)(b.cols_p / V);
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < chunks_total; q += (int64_t)gridDim.x * 256) {
        const bool first = q < chunks_a;
        const int64_t local = first ? q : q - chunks_a;
        const T* src = static_cast<const T*>(first ? a.src : b.src);
        T* dst = static_cast<T*>(first ? a.dst : b.dst);
        const int64_t ld = first ? a.ld : b.ld;
        const int rows = first ? a.rows : b.rows, cols = first ? a.cols : b.cols;
        const int64_t cols_p = first ? a.cols_p : b.cols_p;
        const int64_t per_row = cols_p / V;
        const int64_t r = chunk_row(local, per_row, first ? inv_a : inv_b);
        const int c0 = (int)(local - r * per_row) * V;
        T v[V];
        if (r < rows && c0 + V <= cols) {
            // a whole chunk inside the source: one 16-byte load from an address that
            // is only element-aligned
            load16(v, src + r * ld + c0);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = (r < rows && c0 + e < cols) ? src[r * ld + c0 + e] : T(0);
        }
        *reinterpret_cast<u32x4*>(dst + r * cols_p + c0) = *reinterpret_cast<const u32x4*>(v);
    }
}

int launch_pack(int elem_size, const PackJob& a, const PackJob& b, hipStream_t stream) {
    const int V = 16 / elem_size;
    const int64_t chunks_a = (int64_t)a.rows_p * a.cols_p / V;
    const int64_t total = chunks_a + (int64_t)b.rows_p * b.cols_p / V;
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 8192));
    if (elem_size == 2) return launch_status(pack_pad<uint16_t>, dim3(grid), dim3(256), stream, a, b, chunks_a, total);
    return launch_status(pack_pad<float>, dim3(grid), dim3(256), stream, a, b, chunks_a, total);
}

}  // namespace dg
