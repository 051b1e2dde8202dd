// plan.h -- internal interface between the C ABI and the host-only planner.
#pragma once
#include <stdint.h>

#include "../../include/gemm.h"
#include "menu.h"

namespace dg {

extern const MenuEntry kMenu[kMenuSize];

void set_error(const char* fmt, ...);
void clear_error();
const char* last_error();

// True when a rows x cols matrix with leading dimension ld (elements of up to 4
// bytes) spans fewer than 2^62 bytes, so 64-bit extents and offsets cannot overflow.
bool extent_fits(int64_t rows, int64_t cols, int64_t ld);
int validate(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
             int dtype);
// ws_bytes: workspace available for split K or packing (0: neither).
// fused_epilogue: the call applies an epilogue (only epilogue_capable kernels).
int plan(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
         uintptr_t a, uintptr_t b, uintptr_t c, int num_cus, const char* arch, int64_t ws_bytes,
         bool fused_epilogue, const gemm_config* req, gemm_config* out);
int menu_entry(int index, int* variant, int* dtype, int* opb, gemm_config* out);

// Packed-operand layout: A padded to Mp x Kp, B to Kp x Np (row-major) or Np x Kp
// (column-major); Mp, Np multiples of 256, Kp of 64. A's copy starts the
// workspace, B's follows at pack_a_bytes (a multiple of 256).
void pack_dims(int64_t M, int64_t N, int64_t K, int64_t* Mp, int64_t* Np, int64_t* Kp);
int64_t pack_a_bytes(int dtype, int64_t M, int64_t N, int64_t K);
int64_t pack_workspace(int opB, int dtype, int64_t M, int64_t N, int64_t K);

// Validation of one grouped entry (the gemm_ex rules plus batch and strides).
int validate_problem(int opA, int opB, int dtype, const gemm_problem& p, int index);
// Tile-row group size the planner uses for a problem of tiles_m x tiles_n tiles.
int default_group_m(int64_t tiles_m, int64_t tiles_n);
int plan_grouped(int opA, int opB, int dtype, const gemm_problem* probs, int count, int num_cus, const char* arch,
                 const gemm_config* req, gemm_config* out);

}  // namespace dg
