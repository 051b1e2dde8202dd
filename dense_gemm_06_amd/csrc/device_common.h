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
        g.ep.kind = 0;  // partial products are plain fp32; the reduction applies the epilogue
    }
}

// Tile of workgroup blockIdx.x in round r of a grid of G workgroups that walks
// `total` tiles in rounds of G (round r holds tiles r*G .. r*G + R - 1, R = min(G,
// total - r*G)), or -1 when the round has none for it. With xcd_remap (G a multiple
// of 8) the round's tiles are split into 8 contiguous runs of as equal a length as
// possible, run x going to the workgroups of XCD x (hardware id mod 8), so that a
// partial last round still spreads over every XCD and each XCD's tiles stay
// adjacent in raster order. A full round (R = G) gives XCD x the tiles x*G/8 ..
// x*G/8 + G/8 - 1.
__device__ __forceinline__ int round_tile(int r, int total, int xcd_remap) {
    const int G = gridDim.x, bid = blockIdx.x;
    const int base = r * G;
    const int R = min(G, total - base);
    if (!xcd_remap || (G & 7) != 0) return bid < R ? base + bid : -1;
    const int x = bid & 7, local = bid >> 3;
    const int q = R >> 3, rem = R & 7;
    return local < q + (x < rem ? 1 : 0) ? base + x * q + min(x, rem) + local : -1;
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
    g.ep.kind = 0;
}

// ---- epilogue and C stores

// fp32 -> bf16, round to nearest even: the hardware conversion (v_cvt_pk_bf16_f32,
// two values per instruction), which on gfx950 gives the same bits as the integer
// round-to-nearest-even (add 0x7fff plus the kept lowest bit, keep the high half) for
// every one of the 2^32 fp32 patterns except NaNs, which stay NaNs (checked
// exhaustively on the device).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ __forceinline__ float load_out(const void* p, int dt, size_t i) {
    if (dt == DT_F32) return static_cast<const float*>(p)[i];
    const uint16_t h = static_cast<const uint16_t*>(p)[i];
    return dt == DT_F16 ? (float)__builtin_bit_cast(_Float16, h) : __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ void store_out(void* p, int dt, size_t i, float x) {
    if (dt == DT_F32) static_cast<float*>(p)[i] = x;
    else if (dt == DT_F16) static_cast<_Float16*>(p)[i] = (_Float16)x;
    else static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(x);
}

// GELU in its tanh form (Hendrycks and Gimpel): x/2 * (1 + tanh(u)) with
// u = sqrt(2/pi) (x + 0.044715 x^3). Since 1 + tanh(u) = 2 / (1 + e^(-2u)), this
// is x / (1 + e^(-2u)): a hardware exponential and reciprocal, no cancellation for
// large negative u, and exactly x or 0 (of x's sign) where e^(-2u) under- or overflows.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float u2 = 1.5957691216057308f * (x + 0.044715f * x * x * x);  // 2u
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-u2));
}

__device__ __forceinline__ float epilogue_value(const Epilogue& ep, float acc, size_t ri, int n) {
    float x = ep.alpha * acc;
    if (ep.beta != 0.0f) x = fmaf(ep.beta, load_out(ep.R, ep.out_dt, ri), x);
    if (ep.bias) x += ep.bias[n];
    if (ep.act == ACT_RELU) x = x > 0.0f ? x : 0.0f;
    else if (ep.act == ACT_GELU_TANH) x = gelu_tanh(x);
    return x;
}

// The epilogue of one run, out of line: inlined into every run of a kernel's
// unrolled store loop it would make the loop too large to unroll, and the
// accumulators would then be indexed at run time (moved to scratch memory).
// A whole run moves as one vector (16 bytes of fp32, 8 bytes of 16-bit values)
// for both the residual read and the store, at any element-aligned address:
// gfx950 serves under-aligned vector stores as it serves under-aligned loads.
__device__ __forceinline__ f32x4 load_out4(const void* p, int dt, size_t i) {
    if (dt == DT_F32) {
        f32x4 r;
        __builtin_memcpy(&r, static_cast<const float*>(p) + i, 16);
        return r;
    }
    u32x2 w;
    __builtin_memcpy(&w, static_cast<const uint16_t*>(p) + i, 8);
    f32x4 r;
    if (dt == DT_F16) {
        r[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xffffu));
        r[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16));
        r[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xffffu));
        r[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16));
    } else {
        r[0] = __uint_as_float(w[0] << 16);
        r[1] = __uint_as_float(w[0] & 0xffff0000u);
        r[2] = __uint_as_float(w[1] << 16);
        r[3] = __uint_as_float(w[1] & 0xffff0000u);
    }
    return r;
}

__device__ __forceinline__ void store_out4(void* p, int dt, size_t i, f32x4 x) {
    if (dt == DT_F32) {
        __builtin_memcpy(static_cast<float*>(p) + i, &x, 16);
        return;
    }
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        h[e] = dt == DT_F16 ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[e]) : (uint32_t)f32_to_bf16_rne(x[e]);
    const u32x2 w = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    __builtin_memcpy(static_cast<uint16_t*>(p) + i, &w, 8);
}

// Wave-uniform values handed to an out-of-line function arrive in vector registers;
// readfirstlane tells the compiler they are uniform, so branches on them are scalar
// instead of masked. 64-bit values go through two unsigned 32-bit halves.
__device__ __forceinline__ uint32_t uni32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
    return ((uint64_t)uni32((uint32_t)(x >> 32)) << 32) | (uint64_t)uni32((uint32_t)x);
}
__device__ __forceinline__ float unif(float x) { return __uint_as_float(uni32(__float_as_uint(x))); }

// The epilogue of the run C[m][n .. n+3] (columns >= N skipped). A whole run
// moves as one vector for R and for C, and reads bias as one 16-byte load.
__device__ __forceinline__ void epilogue_run4_body(const Epilogue& ep, void* C, int64_t ldc, int N, int m, int n,
                                                   f32x4 v) {
    const size_t ci = (size_t)m * ldc + n, ri = (size_t)m * ep.ldr + n;
    if (n + 4 <= N) {
        const f32x4 r = ep.beta != 0.0f ? load_out4(ep.R, ep.out_dt, ri) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        if (ep.bias) __builtin_memcpy(&b, ep.bias + n, 16);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = ep.alpha * v[e];
            if (ep.beta != 0.0f) t = fmaf(ep.beta, r[e], t);
            t += b[e];
            if (ep.act == ACT_RELU) t = t > 0.0f ? t : 0.0f;
            else if (ep.act == ACT_GELU_TANH) t = gelu_tanh(t);
            x[e] = t;
        }
        store_out4(C, ep.out_dt, ci, x);
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (n + e < N) store_out(C, ep.out_dt, ci + e, epilogue_value(ep, v[e], ri + e, n + e));
}

__device__ __attribute__((noinline)) void epilogue_run4(const Epilogue ep_in, void* C_in, int64_t ldc_in, int N_in,
                                                        int m, int n, f32x4 v) {
    Epilogue ep;
    ep.kind = (int)uni32((uint32_t)ep_in.kind);
    ep.act = (int)uni32((uint32_t)ep_in.act);
    ep.out_dt = (int)uni32((uint32_t)ep_in.out_dt);
    ep.alpha = unif(ep_in.alpha);
    ep.beta = unif(ep_in.beta);
    ep.R = reinterpret_cast<const void*>(uni64(reinterpret_cast<uint64_t>(ep_in.R)));
    ep.ldr = (int64_t)uni64((uint64_t)ep_in.ldr);
    ep.bias = reinterpret_cast<const float*>(uni64(reinterpret_cast<uint64_t>(ep_in.bias)));
    void* C = reinterpret_cast<void*>(uni64(reinterpret_cast<uint64_t>(C_in)));
    const int64_t ldc = (int64_t)uni64((uint64_t)ldc_in);
    const int N = (int)uni32((uint32_t)N_in);
    epilogue_run4_body(ep, C, ldc, N, m, n, v);
}

// Store the run C[m][n .. n+3] (columns >= N skipped; the caller has checked
// m < M). The plain fp32 path uses one 16-byte store when the run is whole, at any
// element-aligned address (gfx950 serves under-aligned vector stores; rows of C
// with an odd leading dimension start at 4-byte offsets); the epilogue path runs
// the out-of-line epilogue. EPI = false compiles the plain path only (kernels
// that never run an epilogue).
template <bool EPI = true>
__device__ __forceinline__ void store_run4(const GemmArgs& g, int m, int n, f32x4 v) {
    if (!EPI || g.ep.kind == 0) {
        float* cp = g.C + (size_t)m * g.ldc + n;
        if (n + 3 < g.N) {
            __builtin_memcpy(cp, &v, 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < g.N) cp[e] = v[e];
        }
        return;
    }
    epilogue_run4(g.ep, g.C, g.ldc, g.N, m, n, v);
}

// Load V consecutive elements starting at p into a register chunk, zero-filling
// the elements at index >= valid (valid <= 0 means the whole chunk is outside
// the matrix and nothing is read). VEC selects one 16-byte load when the chunk
// is complete. The address need only be aligned to the element: gfx950 under the
// HSA runtime serves under-aligned global vector loads (the compiler itself emits
// global_load_dwordx4 for a 16-byte copy from a 2-byte-aligned address there).
template <typename T, int V>
__device__ __forceinline__ void load16(T (&r)[V], const T* p) {
    static_assert(sizeof(T) * V == 16, "a chunk is 16 bytes");
    __builtin_memcpy(r, p, 16);
}
template <typename T, int V, bool VEC>
__device__ __forceinline__ void load_chunk(T (&r)[V], const T* p, int valid) {
    if (VEC && valid >= V) {
        load16(r, p);
    } else if (valid <= 0) {
        // outside the matrix: a branch of its own, so that only lanes whose chunk
        // the edge cuts take the element loads below (and, for 16-bit elements, the
        // wait that packing them needs)
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = T(0);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = (e < valid) ? p[e] : T(0);
    }
}

// An s_waitcnt vmcnt(0) (the other counters untouched) placed where no vector memory
// load is in flight, so that it waits for nothing and tells the compiler's wait
// tracking so. The register-staged kernels call it before an edge k-tile's masked
// loads: their interior and edge load paths meet in one block, the tracking then
// counts the interior path's loads as pending on the edge path as well, and the edge
// path, which reuses those loads' registers as temporaries, waited chunk by chunk for
// its own loads (an edge tile took twice an interior tile's time).
__device__ __forceinline__ void vm_settled() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// As load_chunk for a chunk known to lie inside the matrix: no guards.
template <typename T, int V, bool VEC>
__device__ __forceinline__ void load_chunk_full(T (&r)[V], const T* p) {
    if (VEC) {
        load16(r, p);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = p[e];
    }
}

}  // namespace dg
