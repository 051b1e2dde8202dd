// launch.h -- per-family kernel launchers (one translation unit per family).
#pragma once
#include <hip/hip_runtime.h>

#include "menu.h"

namespace dg {

// Enqueue kernel `id` with `grid` workgroups on `stream`. Returns 0, or -1 if
// `id` does not belong to the family.
int launch_lds_f32(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_f16(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_bf16(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f32(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f16(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_bf16(int id, const GemmArgs& a, unsigned grid, hipStream_t stream);

// Grouped persistent launches (schedule-1 entries only; -1 for any other id).
int launch_lds_f32_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_f16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_lds_bf16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f32_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_f16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);
int launch_mfma_bf16_grouped(int id, const GroupArgs& a, unsigned grid, hipStream_t stream);

}  // namespace dg
