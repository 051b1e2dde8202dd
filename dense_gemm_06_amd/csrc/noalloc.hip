// noalloc.hip -- gemm_ex_noalloc: the product with a workspace that the library
// owns, for callers that cannot allocate device memory themselves (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace is `scratch`, a file-scope device array of GEMM_NOALLOC_SCRATCH_BYTES.
// Every GPU that runs this library holds its own copy of it until the process ends.
// Host code never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address): on the first call on a device, with that device
// current, its address is looked up once with hipGetSymbolAddress and kept per
// device, and that pointer is what the kernels receive, exactly as they receive a
// caller's workspace in gemm_ex_workspace.
//
// What the kernels keep in the workspace (split-K partial planes, packed operand
// copies) is written in full before it is read within the same call, so nothing in
// it has to start at zero. All calls on one GPU share its array: calls that overlap
// in time on one GPU (different streams, or different host threads without ordering)
// race on it and must not be made.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/gemm.h"
#include "plan.h"
#include "product.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // per device; nullptr until looked up

// The device address of this device's copy of `scratch` (looked up once per device).
int scratch_for_device(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            dg::set_error("hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
            return GEMM_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GEMM_OK;
}

}  // namespace

extern "C" int gemm_ex_noalloc(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg,
                               void* stream) {
    dg::clear_error();
    int dev = 0;
    const hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        dg::set_error("hipGetDevice failed: %s", hipGetErrorString(he));
        return GEMM_ERR_DEVICE;
    }
    void* ws = nullptr;
    int st = scratch_for_device(dev, &ws);
    if (st != GEMM_OK) return st;
    st = dg::run_product(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, dg::plain_epilogue(), cfg, ws,
                         GEMM_NOALLOC_SCRATCH_BYTES, stream);
    if (st == GEMM_ERR_INVALID_VALUE && strstr(dg::last_error(), "workspace") != nullptr) {
        // a forced split or packing that needs more than the fixed scratch
        const std::string why = dg::last_error();
        dg::set_error("gemm_ex_noalloc: the library's scratch holds %lld bytes, too few for this request (%s)",
                      (long long)GEMM_NOALLOC_SCRATCH_BYTES, why.c_str());
    }
    return st;
}
