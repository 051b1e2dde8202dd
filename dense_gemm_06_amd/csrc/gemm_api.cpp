// gemm_api.cpp -- the C ABI declared in include/gemm.h.
//
// Validation and planning are host-only (plan.cpp); this file adds the device
// query, the pointer checks and the launch. Every status from the HIP runtime
// is checked and turned into a gemm_status with a description, in the spirit of
// the chapter's runtime that raises on any nonzero driver status and says what
// failed ("GPU architecture and mapping kernels", section 12.10).
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gemm.h"
#include "launch.h"
#include "plan.h"
#include "product.h"

namespace {

struct DeviceInfo {
    bool valid = false;
    int status = GEMM_ERR_DEVICE;
    int num_cus = 0;
    char arch[64] = {0};
};

std::mutex g_dev_mutex;
std::vector<DeviceInfo> g_devs;

// Per-device (CU count, architecture), queried once per device.
int device_info(int dev, DeviceInfo* out) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (dev < 0) {
        dg::set_error("invalid device index %d", dev);
        return GEMM_ERR_DEVICE;
    }
    if ((size_t)dev >= g_devs.size()) g_devs.resize(dev + 1);
    DeviceInfo& d = g_devs[dev];
    if (!d.valid) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            dg::set_error("hipGetDeviceProperties(%d) failed: %s", dev, hipGetErrorString(e));
            return GEMM_ERR_DEVICE;
        }
        d.num_cus = prop.multiProcessorCount;
        strncpy(d.arch, prop.gcnArchName, sizeof d.arch - 1);
        d.valid = true;
    }
    *out = d;
    return GEMM_OK;
}

bool ranges_overlap(uintptr_t a, uint64_t alen, uintptr_t b, uint64_t blen) {
    if (alen == 0 || blen == 0) return false;
    return a < b + blen && b < a + alen;
}

int launch(int id, const dg::GemmArgs& args, unsigned grid, unsigned grid_y, hipStream_t s) {
    const dg::MenuEntry& e = dg::kMenu[id];
    int rc = -1;
    if (e.variant == dg::V_LDS) {
        rc = e.dtype == dg::DT_F32 ? dg::launch_lds_f32(id, args, grid, grid_y, s)
             : e.dtype == dg::DT_F16 ? dg::launch_lds_f16(id, args, grid, grid_y, s)
                                     : dg::launch_lds_bf16(id, args, grid, grid_y, s);
    } else {
        rc = e.dtype == dg::DT_F32 ? dg::launch_mfma_f32(id, args, grid, grid_y, s)
             : e.dtype == dg::DT_F16 ? dg::launch_mfma_f16(id, args, grid, grid_y, s)
                                     : dg::launch_mfma_bf16(id, args, grid, grid_y, s);
    }
    return rc;
}

int launch_grouped(int id, const dg::GroupArgs& args, unsigned grid, hipStream_t s) {
    const dg::MenuEntry& e = dg::kMenu[id];
    if (e.variant == dg::V_LDS) {
        return e.dtype == dg::DT_F32 ? dg::launch_lds_f32_grouped(id, args, grid, s)
               : e.dtype == dg::DT_F16 ? dg::launch_lds_f16_grouped(id, args, grid, s)
                                       : dg::launch_lds_bf16_grouped(id, args, grid, s);
    }
    return e.dtype == dg::DT_F32 ? dg::launch_mfma_f32_grouped(id, args, grid, s)
           : e.dtype == dg::DT_F16 ? dg::launch_mfma_f16_grouped(id, args, grid, s)
                                   : dg::launch_mfma_bf16_grouped(id, args, grid, s);
}

// A launcher's result as a gemm_status: -1 means the kernel id has no launcher
// (an internal inconsistency), a positive value is the hipError_t of the launch.
int launch_result(int rc, const char* what, int id) {
    if (rc == 0) return GEMM_OK;
    if (rc < 0) dg::set_error("internal: %s %d has no launcher", what, id);
    else dg::set_error("%s %d: launch failed: %s", what, id, hipGetErrorString((hipError_t)rc));
    return GEMM_ERR_LAUNCH;
}

// Byte extent of `batch` matrices of rows x cols (leading dimension ld) placed
// `stride` elements apart, or 0 when it does not fit in the address space.
uint64_t extent(int64_t batch, int64_t stride, int64_t rows, int64_t cols, int64_t ld, int64_t es) {
    const unsigned __int128 n = (unsigned __int128)(batch - 1) * (uint64_t)stride + (unsigned __int128)(rows - 1) * (uint64_t)ld +
                                (uint64_t)cols;
    const unsigned __int128 bytes = n * (uint64_t)es;
    return bytes >> 62 ? 0 : (uint64_t)bytes;
}

}  // namespace

extern "C" {

int gemm_grouped(int opA, int opB, int dtype, const gemm_problem* problems, int count, const gemm_config* cfg,
                 void* stream) {
    dg::clear_error();
    if (count < 0) {
        dg::set_error("count = %d must be non-negative", count);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (count == 0) return GEMM_OK;
    if (problems == nullptr) {
        dg::set_error("problems is NULL with count = %d", count);
        return GEMM_ERR_NULL_POINTER;
    }
    struct Range { uintptr_t lo; uint64_t len; int index; };
    std::vector<Range> outs, ins;
    const int64_t es = dtype == GEMM_F32 ? 4 : 2;
    int with_work = 0;
    for (int i = 0; i < count; ++i) {
        const gemm_problem& p = problems[i];
        int st = dg::validate_problem(opA, opB, dtype, p, i);
        if (st != GEMM_OK) return st;
        if (p.M == 0 || p.N == 0 || p.batch == 0) continue;
        if (p.batch >= ((int64_t)1 << 31)) {
            dg::set_error("problem %d: batch = %lld must be below 2^31", i, (long long)p.batch);
            return GEMM_ERR_UNSUPPORTED;
        }
        if (p.C == nullptr || (p.K > 0 && (p.A == nullptr || p.B == nullptr))) {
            dg::set_error("problem %d: NULL operand: A = %p, B = %p, C = %p (M = %lld, N = %lld, K = %lld)", i, p.A,
                          p.B, (void*)p.C, (long long)p.M, (long long)p.N, (long long)p.K);
            return GEMM_ERR_NULL_POINTER;
        }
        const uint64_t clen = extent(p.batch, p.stride_c, p.M, p.N, p.ldc, 4);
        uint64_t alen = 1, blen = 1;
        if (p.K > 0) {
            alen = extent(p.batch, p.stride_a, p.M, p.K, p.lda, es);
            blen = opB == GEMM_OP_N ? extent(p.batch, p.stride_b, p.K, p.N, p.ldb, es)
                                    : extent(p.batch, p.stride_b, p.N, p.K, p.ldb, es);
        }
        if (clen == 0 || alen == 0 || blen == 0) {
            dg::set_error("problem %d: the operands' address ranges do not fit in 64 bits", i);
            return GEMM_ERR_INVALID_VALUE;
        }
        outs.push_back({(uintptr_t)p.C, clen, i});
        if (p.K > 0) {
            ins.push_back({(uintptr_t)p.A, alen, i});
            ins.push_back({(uintptr_t)p.B, blen, i});
        }
        ++with_work;
    }
    if (with_work == 0) return GEMM_OK;
    for (size_t o = 0; o < outs.size(); ++o) {
        for (const Range& r : ins)
            if (ranges_overlap(outs[o].lo, outs[o].len, r.lo, r.len)) {
                dg::set_error("the output of problem %d overlaps an input of problem %d", outs[o].index, r.index);
                return GEMM_ERR_INVALID_VALUE;
            }
        for (size_t q = o + 1; q < outs.size(); ++q)
            if (ranges_overlap(outs[o].lo, outs[o].len, outs[q].lo, outs[q].len)) {
                dg::set_error("the outputs of problems %d and %d overlap", outs[o].index, outs[q].index);
                return GEMM_ERR_INVALID_VALUE;
            }
    }
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        dg::set_error("hipGetDevice failed: %s", hipGetErrorString(he));
        return GEMM_ERR_DEVICE;
    }
    DeviceInfo info;
    int st = device_info(dev, &info);
    if (st != GEMM_OK) return st;
    gemm_config plan;
    st = dg::plan_grouped(opA, opB, dtype, problems, count, info.num_cus, info.arch, cfg, &plan);
    if (st != GEMM_OK) return st;

    // segment tables, at most kMaxGroupSegments per launch
    std::vector<dg::GroupArgs> launches;
    for (int i = 0; i < count; ++i) {
        const gemm_problem& p = problems[i];
        if (p.M == 0 || p.N == 0 || p.batch == 0) continue;
        if (launches.empty() || launches.back().count == dg::kMaxGroupSegments) {
            launches.emplace_back();
            dg::GroupArgs& a = launches.back();
            memset(&a, 0, sizeof a);
        }
        dg::GroupArgs& a = launches.back();
        dg::GroupSeg& sg = a.seg[a.count++];
        sg.A = p.A;
        sg.B = p.B;
        sg.C = p.C;
        sg.sa = p.stride_a;
        sg.sb = p.stride_b;
        sg.sc = p.stride_c;
        sg.lda = (int)p.lda;
        sg.ldb = (int)p.ldb;
        sg.ldc = (int)p.ldc;
        sg.M = (int)p.M;
        sg.N = (int)p.N;
        sg.K = (int)p.K;
        sg.batch = (int)p.batch;
        sg.tiles_m = (int)((p.M + plan.bm - 1) / plan.bm);
        sg.tiles_n = (int)((p.N + plan.bn - 1) / plan.bn);
        const int gm = plan.group_m ? plan.group_m : dg::default_group_m(sg.tiles_m, sg.tiles_n);
        sg.group_m = std::max(1, std::min(gm, sg.tiles_m));
        sg.tile_begin = a.total_tiles;
        a.total_tiles += sg.batch * sg.tiles_m * sg.tiles_n;  // < 2^31 in total (checked by the planner)
    }
    for (dg::GroupArgs& a : launches) {
        const unsigned grid = (unsigned)std::min<int64_t>(a.total_tiles, plan.grid);
        a.xcd_remap = plan.xcd_remap;
        st = launch_result(launch_grouped(plan.kernel_id, a, grid, (hipStream_t)stream), "grouped kernel",
                           plan.kernel_id);
        if (st != GEMM_OK) return st;
    }
    return GEMM_OK;
}

int gemm_grouped_plan(int opA, int opB, int dtype, const gemm_problem* problems, int count, int num_cus,
                      const char* arch, const gemm_config* request, gemm_config* out) {
    dg::clear_error();
    if (out == nullptr) {
        dg::set_error("gemm_grouped_plan: out is NULL");
        return GEMM_ERR_NULL_POINTER;
    }
    return dg::plan_grouped(opA, opB, dtype, problems, count, num_cus, arch, request, out);
}

int gemm_strided_batched(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b, float* C, int64_t ldc,
                         int64_t stride_c, int64_t batch, int dtype, const gemm_config* cfg, void* stream) {
    gemm_problem p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = A;
    p.lda = lda;
    p.stride_a = stride_a;
    p.B = B;
    p.ldb = ldb;
    p.stride_b = stride_b;
    p.C = C;
    p.ldc = ldc;
    p.stride_c = stride_c;
    p.batch = batch;
    return gemm_grouped(opA, opB, dtype, &p, 1, cfg, stream);
}

}  // extern "C"

namespace dg {

int run_product(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, void* C, int64_t ldc, int dtype, const dg::Epilogue& ep, const gemm_config* cfg,
                void* workspace, int64_t workspace_bytes, void* stream) {
    int st = dg::validate(opA, opB, M, N, K, lda, ldb, ldc, dtype);
    if (st != GEMM_OK) return st;
    if (workspace_bytes < 0) {
        dg::set_error("workspace_bytes = %lld must be non-negative", (long long)workspace_bytes);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (workspace_bytes > 0 && workspace == nullptr) {
        dg::set_error("workspace is NULL with workspace_bytes = %lld", (long long)workspace_bytes);
        return GEMM_ERR_NULL_POINTER;
    }
    if (M == 0 || N == 0) return GEMM_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) {
        dg::set_error("NULL operand: A = %p, B = %p, C = %p (M = %lld, N = %lld, K = %lld)", A, B, C,
                      (long long)M, (long long)N, (long long)K);
        return GEMM_ERR_NULL_POINTER;
    }
    const uint64_t es = dtype == GEMM_F32 ? 4 : 2;
    const uint64_t ces = (ep.kind == 0 || ep.out_dt == dg::DT_F32) ? 4 : 2;
    const uint64_t clen = ((uint64_t)(M - 1) * ldc + N) * ces;
    const uint64_t alen = K > 0 ? ((uint64_t)(M - 1) * lda + K) * es : 0;
    const uint64_t blen =
        K > 0 ? (opB == GEMM_OP_N ? (uint64_t)(K - 1) * ldb + N : (uint64_t)(N - 1) * ldb + K) * es : 0;
    if (ranges_overlap((uintptr_t)C, clen, (uintptr_t)A, alen) ||
        ranges_overlap((uintptr_t)C, clen, (uintptr_t)B, blen)) {
        dg::set_error("C overlaps A or B; the output must not alias an input");
        return GEMM_ERR_INVALID_VALUE;
    }
    // epilogue operands: R (C itself, or disjoint from C) and bias (disjoint from C)
    const uint64_t rlen = (ep.kind != 0 && ep.beta != 0.0f) ? ((uint64_t)(M - 1) * ep.ldr + N) * ces : 0;
    const uint64_t biaslen = (ep.kind != 0 && ep.bias) ? (uint64_t)N * 4 : 0;
    if (rlen && !((uintptr_t)ep.R == (uintptr_t)C && ep.ldr == ldc) &&
        ranges_overlap((uintptr_t)ep.R, rlen, (uintptr_t)C, clen)) {
        dg::set_error("R overlaps C without being C itself (R == C with ldr == ldc is the in-place form)");
        return GEMM_ERR_INVALID_VALUE;
    }
    if (biaslen && ranges_overlap((uintptr_t)ep.bias, biaslen, (uintptr_t)C, clen)) {
        dg::set_error("bias overlaps C");
        return GEMM_ERR_INVALID_VALUE;
    }
    if (workspace_bytes > 0) {
        // the whole declared workspace: aligned, and disjoint from every operand
        const uintptr_t w = (uintptr_t)workspace;
        if ((w & 15) != 0) {
            dg::set_error("the workspace must be 16-byte aligned (got %p)", workspace);
            return GEMM_ERR_INVALID_VALUE;
        }
        const uint64_t wl = (uint64_t)workspace_bytes;
        if (ranges_overlap(w, wl, (uintptr_t)A, alen) || ranges_overlap(w, wl, (uintptr_t)B, blen) ||
            ranges_overlap(w, wl, (uintptr_t)C, clen) || ranges_overlap(w, wl, (uintptr_t)ep.R, rlen) ||
            ranges_overlap(w, wl, (uintptr_t)ep.bias, biaslen)) {
            dg::set_error("the workspace overlaps A, B, C or an epilogue operand");
            return GEMM_ERR_INVALID_VALUE;
        }
    }
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        dg::set_error("hipGetDevice failed: %s", hipGetErrorString(he));
        return GEMM_ERR_DEVICE;
    }
    DeviceInfo info;
    st = device_info(dev, &info);
    if (st != GEMM_OK) return st;
    gemm_config plan;
    st = dg::plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, (uintptr_t)A, (uintptr_t)B, (uintptr_t)C, info.num_cus,
                  info.arch, workspace_bytes, ep.kind != 0, cfg, &plan);
    if (st != GEMM_OK) return st;

    dg::GemmArgs args;
    args.A = A;
    args.B = B;
    args.C = static_cast<float*>(C);
    args.lda = lda;
    args.ldb = ldb;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)plan.tiles_m;
    args.tiles_n = (int)plan.tiles_n;
    args.group_m = plan.group_m;
    args.xcd_remap = plan.xcd_remap;
    args.k_split = plan.split_k;
    args.k_chunk = plan.k_chunk;
    args.work = static_cast<float*>(workspace);
    args.work_ld = (N + 3) / 4 * 4;
    args.work_slice = M * args.work_ld;
    args.ep = ep;
    // stream-K: the tiles past the last whole round of the grid (all of them when
    // there are fewer tiles than workgroups)
    const int64_t tiles_total = plan.tiles_m * plan.tiles_n;
    args.sk_tiles = plan.stream_k == 2 ? (int)(tiles_total > plan.grid ? tiles_total % plan.grid : tiles_total) : 0;
    args.sk_width = plan.stream_k == 2 ? plan.sk_width : 0;
    if (plan.pack == 2) {
        // zero-padded copies of A and B in the workspace, then the product on them
        int64_t Mp, Np, Kp;
        dg::pack_dims(M, N, K, &Mp, &Np, &Kp);
        char* ap = static_cast<char*>(workspace);
        char* bp = ap + dg::pack_a_bytes(dtype, M, N, K);
        dg::PackJob ja{A, ap, lda, (int)M, (int)K, (int)Mp, (int)Kp};
        dg::PackJob jb = opB == GEMM_OP_N ? dg::PackJob{B, bp, ldb, (int)K, (int)N, (int)Kp, (int)Np}
                                          : dg::PackJob{B, bp, ldb, (int)N, (int)K, (int)Np, (int)Kp};
        st = launch_result(dg::launch_pack((int)es, ja, jb, (hipStream_t)stream), "packing kernel", 0);
        if (st != GEMM_OK) return st;
        args.A = ap;
        args.B = bp;
        args.lda = Kp;
        args.ldb = opB == GEMM_OP_N ? Np : Kp;
        args.K = (int)Kp;
    }
    st = launch_result(launch(plan.kernel_id, args, (unsigned)plan.grid, (unsigned)plan.split_k, (hipStream_t)stream),
                       "kernel", plan.kernel_id);
    if (st != GEMM_OK) return st;
    if (plan.split_k > 1)
        return launch_result(dg::launch_splitk_reduce(args.work, plan.split_k, args.work_slice, args.work_ld, (int)M,
                                                      (int)N, C, ldc, ep, (hipStream_t)stream),
                             "split-K reduction kernel", 0);
    if (args.sk_tiles > 0)
        return launch_result(dg::launch_streamk_fixup(args.work, args.sk_width, args.sk_tiles, args.K / plan.bk,
                                                      (int)(tiles_total - args.sk_tiles), args.tiles_m, args.tiles_n,
                                                      args.group_m, (int)M, (int)N, C, ldc, ep, (hipStream_t)stream),
                             "stream-K fixup kernel", 0);
    return GEMM_OK;
}

Epilogue plain_epilogue() {
    Epilogue ep;
    memset(&ep, 0, sizeof ep);
    ep.alpha = 1.0f;
    return ep;
}

}  // namespace dg

namespace {

using dg::plain_epilogue;
using dg::run_product;

// gemm_epilogue -> the kernels' descriptor; an identity epilogue (alpha 1, no
// residual, no bias, no activation, fp32 C) becomes the plain store.
int to_epilogue(const gemm_epilogue* e, dg::Epilogue* out) {
    *out = plain_epilogue();
    if (e == nullptr) return GEMM_OK;
    if (e->out_dtype < GEMM_F32 || e->out_dtype > GEMM_BF16) {
        dg::set_error("epilogue out_dtype %d is not GEMM_F32, GEMM_F16 or GEMM_BF16", e->out_dtype);
        return GEMM_ERR_INVALID_VALUE;
    }
    if (e->activation < GEMM_ACT_NONE || e->activation > GEMM_ACT_GELU_TANH) {
        dg::set_error("epilogue activation %d is not a gemm_activation", e->activation);
        return GEMM_ERR_INVALID_VALUE;
    }
    const bool identity = e->alpha == 1.0f && e->beta == 0.0f && e->bias == nullptr &&
                          e->activation == GEMM_ACT_NONE && e->out_dtype == GEMM_F32;
    if (identity) return GEMM_OK;
    out->kind = 1;
    out->act = e->activation;
    out->out_dt = e->out_dtype;
    out->alpha = e->alpha;
    out->beta = e->beta;
    out->R = e->R;
    out->ldr = e->ldr;
    out->bias = e->bias;
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_ex_workspace(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      const void* B, int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg,
                      void* workspace, int64_t workspace_bytes, void* stream) {
    dg::clear_error();
    return run_product(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, plain_epilogue(), cfg, workspace,
                       workspace_bytes, stream);
}

int gemm_ex_epilogue(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, int dtype, const gemm_epilogue* epilogue,
                     const gemm_config* cfg, void* workspace, int64_t workspace_bytes, void* stream) {
    dg::clear_error();
    dg::Epilogue ep;
    int st = to_epilogue(epilogue, &ep);
    if (st != GEMM_OK) return st;
    if (ep.kind != 0 && ep.beta != 0.0f && M > 0 && N > 0) {
        if (ep.R == nullptr) {
            dg::set_error("epilogue beta = %g needs R, which is NULL", (double)ep.beta);
            return GEMM_ERR_NULL_POINTER;
        }
        if (ep.ldr < std::max<int64_t>(1, N)) {
            dg::set_error("epilogue ldr = %lld is smaller than max(1, N) = %lld", (long long)ep.ldr,
                          (long long)std::max<int64_t>(1, N));
            return GEMM_ERR_INVALID_VALUE;
        }
        if (!dg::extent_fits(M, N, ep.ldr)) {
            dg::set_error("epilogue ldr = %lld: R's extent (M - 1) * ldr + N (M = %lld, N = %lld) does not fit in "
                          "the address space", (long long)ep.ldr, (long long)M, (long long)N);
            return GEMM_ERR_INVALID_VALUE;
        }
    }
    return run_product(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, ep, cfg, workspace, workspace_bytes,
                       stream);
}

int gemm_ex(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
            int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg, void* stream) {
    return gemm_ex_workspace(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, cfg, nullptr, 0, stream);
}

int gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
         int64_t ldc, int dtype, void* stream) {
    return gemm_ex(GEMM_OP_N, GEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, dtype, nullptr, stream);
}

int gemm_plan(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
              uintptr_t a_addr, uintptr_t b_addr, uintptr_t c_addr, int num_cus, const char* arch,
              const gemm_config* request, gemm_config* out) {
    dg::clear_error();
    if (out == nullptr) {
        dg::set_error("gemm_plan: out is NULL");
        return GEMM_ERR_NULL_POINTER;
    }
    return dg::plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr, b_addr, c_addr, num_cus, arch, 0, false,
                    request, out);
}

int gemm_plan_workspace(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                        int dtype, uintptr_t a_addr, uintptr_t b_addr, uintptr_t c_addr, int num_cus,
                        const char* arch, int64_t workspace_bytes, const gemm_epilogue* epilogue,
                        const gemm_config* request, gemm_config* out) {
    dg::clear_error();
    if (out == nullptr) {
        dg::set_error("gemm_plan_workspace: out is NULL");
        return GEMM_ERR_NULL_POINTER;
    }
    dg::Epilogue ep;
    const int st = to_epilogue(epilogue, &ep);
    if (st != GEMM_OK) return st;
    return dg::plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr, b_addr, c_addr, num_cus, arch,
                    workspace_bytes, ep.kind != 0, request, out);
}

int gemm_menu_size(void) { return dg::kMenuSize; }

int gemm_menu_entry(int index, int* variant, int* dtype, int* opb, gemm_config* out) {
    dg::clear_error();
    return dg::menu_entry(index, variant, dtype, opb, out);
}

int gemm_device_info(int device, int* num_cus, char* arch, int len) {
    dg::clear_error();
    DeviceInfo info;
    int st = device_info(device, &info);
    if (st != GEMM_OK) return st;
    if (num_cus) *num_cus = info.num_cus;
    if (arch && len > 0) {
        strncpy(arch, info.arch, (size_t)len - 1);
        arch[len - 1] = '\0';
    }
    return GEMM_OK;
}

const char* gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: an argument is out of range";
        case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER: a required operand pointer is NULL";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: valid request not implemented by this build";
        case GEMM_ERR_DEVICE: return "GEMM_ERR_DEVICE: no usable gfx950 device";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: the kernel launch failed";
        default: return "unknown gemm_status";
    }
}

const char* gemm_last_error(void) { return dg::last_error(); }

}  // extern "C"
