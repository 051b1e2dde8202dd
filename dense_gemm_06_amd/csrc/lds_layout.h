// lds_layout.h -- LDS layouts (XOR chunk swizzles) shared by the kernels, and
// address-space casts for direct global -> LDS copies.
#pragma once
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

// 64-byte k-major rows read 16 rows at a time (16x16x32 fragments): chunk c of row
// r is stored at c ^ ((r >> 1) & 3), which keeps the 16-byte fragment reads (16
// rows x 4 chunks) conflict-free under the phase rule above.
__device__ __forceinline__ int kmaj64_swz(int r) { return (r >> 1) & 3; }

// 64-byte k-major rows read 32 rows at a time and 512-byte n-major rows read as 4
// rows x 64 bytes per 32-lane transpose phase (32x32x16 fragments): the chunk
// swizzles below are conflict-free under the same rules.
__device__ __forceinline__ int kmaj32_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int nmaj32_swz(int k) { return (k & 3) << 2; }

#define DG_GLB(p) ((__attribute__((address_space(1))) void*)(p))
#define DG_LDSV(p) ((__attribute__((address_space(3))) void*)(p))

}  // namespace dg
