// product.h -- internal: the product with every option, shared by the C entry points.
#pragma once
#include <stdint.h>

#include "../../include/gemm.h"
#include "menu.h"

namespace dg {

// C = A @ B, C of element type ep.out_dt when ep.kind != 0, with an optional
// workspace (split K or packing) and an optional fused epilogue. Every argument is
// validated before the first launch. Returns a gemm_status; the thread's error text
// describes a failure.
int run_product(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, void* C, int64_t ldc, int dtype, const Epilogue& ep, const gemm_config* cfg,
                void* workspace, int64_t workspace_bytes, void* stream);

// The identity epilogue (plain fp32 store of the product).
Epilogue plain_epilogue();

}  // namespace dg
