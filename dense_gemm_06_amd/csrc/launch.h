// launch.h -- per-family kernel launchers (one translation unit per family).
#pragma once
#include <hip/hip_runtime.h>

#include "menu.h"

namespace dg {

template <typename T> struct same_type { typedef T type; };

// Enqueue kernel `fn` with the given by-value arguments and return this launch's
// own status: 0, or the hipError_t the launch reported. A status left over from
// earlier, unrelated work of the calling thread is neither read nor cleared.
template <typename... P>
int launch_status(void (*fn)(P...), dim3 grid, dim3 block, hipStream_t stream, typename same_type<P>::type... a) {
    void* args[] = {static_cast<void*>(&a)...};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, 0, stream);
}

// The family launchers return 0 after enqueueing, -1 if the kernel id has no
// launcher there (it does not belong to the family or cannot split), or the
// positive hipError_t of a launch the runtime refused.

// Enqueue kernel `id` with grid (grid, grid_y) on `stream`; grid_y > 1 is a
// split-K launch (register-staged kernels only).
int launch_lds_f32(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);
int launch_lds_f16(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);
int launch_lds_bf16(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);
int launch_mfma_f32(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);
int launch_mfma_f16(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);
int launch_mfma_bf16(int id, const GemmArgs& a, unsigned grid, unsigned grid_y, hipStream_t stream);

// Grouped persistent launches (schedule-1 entries only; -1 for any other id).
int launch_lds_f32_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_f16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_bf16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f32_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_bf16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);

// Zero-padded copies of A and B in one launch (elem_size 2 or 4).
int launch_pack(int elem_size, const PackJob& a, const PackJob& b, hipStream_t stream);

// C[i][j] = sum over s = 0..S-1, in that order, of work[s * slice + i * work_ld + j]
// for i < M, j < N: the fixed-order reduction of a split-K launch, followed by the
// fused epilogue when ep.kind != 0 (C then has element type ep.out_dt).
int launch_splitk_reduce(const float* work, int S, int64_t slice, int64_t work_ld, int M, int N, void* C,
                         int64_t ldc, const Epilogue& ep, hipStream_t stream);

// Stream-K fixup of a persistent launch on `G` workgroups whose last S tiles (from
// linear tile tile0 on, KT k-tiles each) were dealt out as k-tile shares: every
// tail tile that more than one workgroup worked on gets the sum of its partial sums
// (work slots 2w + p, in k order), through the fused epilogue when ep.kind != 0.
int launch_streamk_fixup(const float* work, int G, int S, int KT, int tile0, int tiles_m, int tiles_n, int group_m,
                         int M, int N, void* C, int64_t ldc, const Epilogue& ep, hipStream_t stream);

}  // namespace dg
