// kernels.h -- the GEMM kernels, C = A @ B with fp32 accumulation, for gfx950.
//
// Two kernel families, both built on the block tiling of "Shared memory and
// tensor cores" (section 13.3: a block stages a tile of A and of B in on-chip
// memory, waits at a barrier, reuses the tiles from there, and waits again
// before they are overwritten) and on the refinements listed in its section
// 13.10 (double buffering, 16-byte global loads, swizzled shared layouts, warp
// (wave) tiling):
//
//   lds_gemm    -- the LDS-staged SIMT kernel: each of 256 threads owns a
//                  register micro-tile (section 13.7) and does fp32 FMAs.
//   mfma16_gemm -- fp16/bf16 inputs on v_mfma_f32_16x16x32_{f16,bf16}, the
//                  CDNA4 counterpart of the chapter's 16x16x16 tensor-core
//                  operation (section 13.8: products exact, sums in fp32).
//   mfma32_gemm -- fp32 inputs on v_mfma_f32_16x16x4_f32 (full fp32 products
//                  and sums; gfx950 has no reduced-precision fp32 matrix op).
//
// Common structure: two LDS stages; the next k-tile is loaded from global memory
// into registers before the current one is consumed and written to the other
// stage afterwards, so one barrier per k-tile separates the write of a stage
// from its reads (read-after-write) and the reads of a stage from its next
// overwrite (write-after-read). Every thread of a workgroup reaches every
// barrier: edge handling is done by zero-filled loads and guarded stores, never
// by an early exit.
//
// Edges: loads of elements outside the matrix (row >= M or N, k >= K) return
// zero and are never dereferenced; stores outside C are skipped. The VEC
// template flag selects 16-byte global loads (requires 16-byte aligned bases
// and leading dimensions that are multiples of 16 bytes; the host checks) and
// otherwise element-wise loads.
#pragma once
#include "kernel_lds.h"
#include "kernel_mfma.h"
#include "kernel_pp.h"
#include "kernel_sp.h"
#include "kernel_f32dc.h"
