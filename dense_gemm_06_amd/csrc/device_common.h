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

// Raster of tile `bid` inside one problem of tiles_m x tiles_n tiles: groups of
// `group_m` tile rows walked column by column (as tile_coords without the XCD
// renumbering).
__device__ __forceinline__ void raster(int bid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int per_group = group_m * tiles_n;
    const int group = bid / per_group;
    const int first_m = group * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int in_group = bid - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
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
    raster(bid, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
}

// Narrow the arguments to this workgroup's K slice (grid y) of a split-K launch:
// A and B advance by the slice's first k, K becomes the slice length, and the
// output is the slice's plane of the workspace. ES is the input element size.
template <int ES, int OPB>
__device__ __forceinline__ void k_slice(GemmArgs& g) {
    if (g.k_split > 1) {
        const int s = blockIdx.y;
        const int kbeg = s * g.k_chunk;
        g.A = static_cast<const char*>(g.A) + (size_t)kbeg * ES;
        g.B = static_cast<const char*>(g.B) + (OPB == 0 ? (size_t)kbeg * (size_t)g.ldb : (size_t)kbeg) * ES;
        g.K = min(g.K - kbeg, g.k_chunk);
        g.C = g.work + (size_t)s * (size_t)g.work_slice;
        g.ldc = g.work_ld;
    }
}

// Persistent workgroup number of this workgroup: with xcd_remap the ids are
// renumbered so that the workgroups of one XCD (hardware id mod 8) get a
// contiguous block of numbers, hence tiles that are adjacent in linear order.
__device__ __forceinline__ int persistent_id(int xcd_remap) {
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if (xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    return bid;
}

// Linear tile t of a grouped launch -> the problem's arguments and tile
// coordinates. The segment search is a short scalar loop over the table (the
// role of the README's prefix-sum search in its grouped scheduler); ES is the
// input element size in bytes.
template <int ES>
__device__ __forceinline__ void group_tile(const GroupArgs& ga, int t, GemmArgs& g, int& tm, int& tn) {
    int s = 0;
    while (s + 1 < ga.count && t >= ga.seg[s + 1].tile_begin) ++s;
    const GroupSeg& sg = ga.seg[s];
    const int per = sg.tiles_m * sg.tiles_n;
    const int local = t - (int)sg.tile_begin;
    const int b = local / per;
    raster(local - b * per, sg.tiles_m, sg.tiles_n, sg.group_m, tm, tn);
    g.A = static_cast<const char*>(sg.A) + (size_t)b * (size_t)sg.sa * ES;
    g.B = static_cast<const char*>(sg.B) + (size_t)b * (size_t)sg.sb * ES;
    g.C = sg.C + (size_t)b * (size_t)sg.sc;
    g.lda = sg.lda;
    g.ldb = sg.ldb;
    g.ldc = sg.ldc;
    g.M = sg.M;
    g.N = sg.N;
    g.K = sg.K;
    g.tiles_m = sg.tiles_m;
    g.tiles_n = sg.tiles_n;
    g.group_m = sg.group_m;
    g.xcd_remap = 0;
    g.k_split = 1;
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
