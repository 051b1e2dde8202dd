// device_common.h -- device-side helpers shared by the GEMM kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "menu.h"

namespace dg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// operand type of the LDS transpose reads
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

#define DG_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Input element storage: fp32 as float, fp16/bf16 as raw 16-bit patterns.
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { typedef float type; static constexpr int vec = 4; };
template <> struct Elem<DT_F16> { typedef uint16_t type; static constexpr int vec = 8; };
template <> struct Elem<DT_BF16> { typedef uint16_t type; static constexpr int vec = 8; };

template <int DT> __device__ __forceinline__ float decode(typename Elem<DT>::type x);
template <> __device__ __forceinline__ float decode<DT_F32>(float x) { return x; }
template <> __device__ __forceinline__ float decode<DT_F16>(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
}
template <> __device__ __forceinline__ float decode<DT_BF16>(uint16_t x) {
    return __uint_as_float((uint32_t)x << 16);
}

// Map a linear workgroup id to a (tile row, tile column).
//
// Workgroups are handed to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2. With xcd_remap the ids are renumbered so that each XCD receives
// a contiguous run of logical tiles; the logical order then walks groups of
// `group_m` tile rows column by column, so the tiles resident on one XCD at the
// same time share a few A row-panels and B column-panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int& tm, int& tn) {
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if (g.xcd_remap && (nblk & 7) == 0) {
        const int per = nblk >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    const int gm = g.group_m;
    const int per_group = gm * g.tiles_n;
    const int group = bid / per_group;
    const int first_m = group * gm;
    const int rows = min(g.tiles_m - first_m, gm);
    const int in_group = bid - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// Load V consecutive elements starting at p into a register chunk, zero-filling
// the elements at index >= valid (valid <= 0 means the whole chunk is outside
// the matrix and nothing is read). VEC selects one 16-byte load when the chunk
// is complete; the caller guarantees 16-byte alignment in that case.
template <typename T, int V, bool VEC>
__device__ __forceinline__ void load_chunk(T (&r)[V], const T* p, int valid) {
    if (VEC && valid >= V) {
        *reinterpret_cast<u32x4*>(r) = *reinterpret_cast<const u32x4*>(p);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = (e < valid) ? p[e] : T(0);
    }
}

// As load_chunk for a chunk known to lie inside the matrix: no guards.
template <typename T, int V, bool VEC>
__device__ __forceinline__ void load_chunk_full(T (&r)[V], const T* p) {
    if (VEC) {
        *reinterpret_cast<u32x4*>(r) = *reinterpret_cast<const u32x4*>(p);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = p[e];
    }
}

}  // namespace dg
