/*
 * gemm.h -- C ABI of the MI355X (gfx950) dense GEMM library.
 *
 * The library computes the dense matrix product C = A @ B, the operation of
 * "Shared memory and tensor cores" (ML compiler from scratch, chapter 13):
 * section 13.1 sets up C = A @ B and its memory traffic, section 13.3 the
 * block-tiled shared-memory kernel, section 13.8 the tensor-core contract
 * (16-bit inputs, products exact, accumulation in fp32). Two kernel families
 * implement it on gfx950: an LDS-staged SIMT kernel and a matrix-core (MFMA)
 * kernel; a heuristic picks one per call (the role of gpu_opt_choice in
 * "GPU architecture and mapping kernels", section 12.9).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - C[i][j] = sum_{k<K} A(i,k) * B(k,j) for 0 <= i < M, 0 <= j < N, accumulated
 *    in fp32, written to C in fp32. C is overwritten: there is no alpha or beta,
 *    and prior contents (NaN included) are ignored.
 *  - Storage is row-major with BLAS-style leading dimensions in ELEMENTS:
 *      A(i,k) = A[i*lda + k]                      (opA = GEMM_OP_N, lda >= max(1,K))
 *      B(k,j) = B[k*ldb + j]                      (opB = GEMM_OP_N, ldb >= max(1,N))
 *      B(k,j) = B[j*ldb + k]  (column-major B)    (opB = GEMM_OP_T, ldb >= max(1,K))
 *      C[i][j] = C[i*ldc + j]                     (ldc >= max(1,N))
 *    Column-major B is the layout the learn-cutedsl README's naive kernel reads
 *    (B indexed as [column, k]) and the one its layout section calls typical.
 *  - dtype gives the element type of A and B: GEMM_F32 (IEEE binary32),
 *    GEMM_F16 (IEEE binary16), GEMM_BF16 (bfloat16). C is fp32 (a fused
 *    epilogue, gemm_ex_epilogue, may store it as fp16 or bf16).
 *  - Pointers A, B, C are DEVICE pointers (memory the caller allocated on the
 *    current HIP device); the caller owns them and the stream. A and B must not
 *    overlap C (the kernels read them through restrict-qualified pointers);
 *    overlap is detected and rejected. No alignment is required: 16-byte global
 *    loads are used only when the bases and leading dimensions allow them.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on
 *    it and the call returns without synchronizing; faults during execution
 *    surface at the caller's next synchronization.
 *  - Degenerate shapes: M == 0 or N == 0 is a successful no-op (nothing is
 *    launched, C untouched); K == 0 writes C[:M,:N] = 0, the empty sum.
 *  - Errors: every argument is validated before anything is enqueued, so a
 *    failing call launches nothing. Calls return a gemm_status; the thread-local
 *    gemm_last_error() describes what was rejected and why. Nothing aborts and
 *    no C++ exception crosses this interface.
 *  - State: the library allocates no device memory and keeps no workspace; the
 *    only state is a per-device cache of (compute-unit count, architecture)
 *    filled on first use, and the fixed scratch array of gemm_ex_noalloc. All
 *    entry points are thread-safe (gemm_ex_noalloc: see its own rule).
 */
#ifndef DENSE_GEMM_06_AMD_GEMM_H
#define DENSE_GEMM_06_AMD_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_F32 = 0, GEMM_F16 = 1, GEMM_BF16 = 2 } gemm_dtype;

typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1, /* negative size, bad enum, short leading dimension, C overlaps A or B */
    GEMM_ERR_NULL_POINTER = 2,  /* NULL operand for a non-empty product */
    GEMM_ERR_UNSUPPORTED = 3,   /* valid request this build does not implement (opA = T, sizes >= 2^31,
                                   a forced configuration that does not exist or does not fit) */
    GEMM_ERR_DEVICE = 4,        /* no HIP device, or the current device is not gfx950 */
    GEMM_ERR_LAUNCH = 5         /* the kernel launch itself failed */
} gemm_status;

typedef enum { GEMM_VARIANT_AUTO = 0, GEMM_VARIANT_LDS = 1, GEMM_VARIANT_MFMA = 2 } gemm_variant;

/*
 * A launch configuration, in the role of the chapter's Opts / launch_dims:
 * which kernel, its tiles, and the grid. As an INPUT (gemm_ex, gemm_plan) only
 * the fields marked "in" are read; 0 / -1 there mean "let the heuristic choose".
 * As an OUTPUT every field describes the launch gemm_ex would make.
 */
typedef struct gemm_config {
    int32_t variant;   /* in/out: gemm_variant (AUTO lets the heuristic choose) */
    int32_t bm, bn;    /* in/out: block tile (0 = any) */
    int32_t bk;        /* out: k depth of one LDS stage */
    int32_t vec;       /* in/out: -1 any, 0 element-wise global loads, 1 16-byte loads */
    int32_t xcd_remap; /* in/out: -1 auto, 0 off, 1 contiguous tile ranges per XCD */
    int32_t group_m;   /* in/out: 0 auto; tile rows per raster group */
    int32_t waves_m, waves_n;   /* in/out: wave grid of an MFMA workgroup (1 x 1 for LDS); 0 = any */
    int32_t thread_m, thread_n; /* out: per-thread micro-tile of the LDS kernel (0 for MFMA) */
    int32_t threads;   /* in/out: 0 any; workgroup size (64 x waves_m x waves_n, or twice that for
                          the fp32 64 x 64 configurations that split K between two wave grids) */
    int32_t lds_bytes; /* out: LDS per workgroup */
    int32_t grid;      /* out: workgroups launched (tiles_m * tiles_n, or a persistent grid) */
    int32_t kernel_id; /* out: index into the library's kernel menu */
    int32_t schedule;  /* in/out: 0 any; 1 register-staged double buffer (any shape); 2 ping-pong
                          with direct global->LDS copies on 16x16x32 MFMAs; 3 not available
                          (requests for it return GEMM_ERR_UNSUPPORTED); 4 ping-pong on 32x32x16
                          MFMAs; 5 software-pipelined 32x32x16 with direct global->LDS copies,
                          4 waves of 128 x 128 or 8 of 128 x 64 (2, 4, 5: MFMA, 16-bit inputs,
                          16-byte aligned operands, any M, and any N for column-major B or N a
                          multiple of 8 for row-major B; 2, 4: K a multiple of 32; 5: K a multiple of 8;
                          4 stores the plain fp32 accumulator only); 6 register-staged with three LDS
                          stages and fragments read half a k-tile ahead (fp32 256 x 128
                          tiles, and 64 x 64 tiles with K over two wave groups; any shape,
                          K not split); 7 the software-pipelined kernel of schedule 5 with
                          register-staged 16-byte loads (16-bit inputs, bases aligned to the
                          element, rows at any offset, any M, K >= 8, any N for column-major
                          B or N >= 8 for row-major B); 8 fp32 64 x 64 tiles with direct
                          global->LDS copies three k-tiles ahead, K over two wave groups
                          (16-byte aligned operands, any M, K a multiple of 64, any N for
                          column-major B or N a multiple of 4 for row-major B; K slices of
                          whole pairs of k-tiles);
                          9 fp32 256 x 128 (three LDS stages) or 128 x 128 (five) tiles on
                          eight waves with direct global->LDS copies (16-byte aligned
                          operands, any M, K a multiple of 32, any N for column-major B or N
                          a multiple of 4 for row-major B) */
    int64_t tiles_m, tiles_n; /* out (grouped: of the first non-empty problem) */
    double est_cycles; /* out: the heuristic's cost estimate (clock cycles) */
    int64_t tiles_total; /* out: output tiles of the call (grouped: of all its problems) */
    int32_t launches;    /* out: kernel launches the call makes */
    int32_t max_grid;    /* in/out: cap on the workgroups of a launch, 0 = heuristic. Grouped calls:
                            the persistent grid. Single calls: a cap below the output tile
                            count selects the persistent form of schedule 5 with 8 waves (each
                            workgroup takes one tile per round of `grid` tiles; K, padded K
                            when packed, a multiple of 32 and at least 128; no split), the only
                            kernel that has one; 0 lets the heuristic use that form with one
                            workgroup per compute unit when the tiles outnumber the compute
                            units; a cap at or above the tile count means one workgroup per tile */
    int32_t split_k;     /* in/out: K slices; in: 0 = heuristic, 1 = no split, S >= 2 = S slices (fewer
                            if K has fewer k-tiles); splitting needs a workspace (gemm_ex_workspace)
                            and one of schedules 1, 5 (not on a persistent grid), 7 (the last
                            slice at least 8 elements of K), 8 (slices of whole pairs of
                            k-tiles, so fewer slices than asked where that rounds up) and 9 */
    int32_t k_chunk;     /* out: K elements per slice (K when not split) */
    int64_t workspace_bytes; /* out: workspace the configuration uses (0 without split or packing) */
    int32_t pack;        /* in/out: operand packing (gemm_ex_workspace); in: 0 = heuristic, 1 = never,
                            2 = always; out: 2 if the call packs, else 1 */
    int32_t stream_k;    /* in/out: stream-K tail on the persistent grid of schedule 5 (8 waves, 16-byte
                            aligned operands, K a multiple of 32 with at least 8 k-tiles, no packing
                            and no split; "Shared memory and tensor cores" section 13.10): the
                            tiles that do not fill a round of `grid` workgroups (all of them when
                            there are fewer tiles than `grid`) are dealt out as equal shares of
                            their k-tiles to sk_width workgroups, whose partial sums a second
                            launch adds in k order. Needs a workspace of sk_width * 512 KiB. in:
                            0 = heuristic, 1 = never, 2 = always (GEMM_ERR_INVALID_VALUE where it
                            cannot apply); out: 2 if the call uses it, else 1 */
    int32_t sk_width;    /* in/out: 0 = heuristic; workgroups the stream-K tail is dealt to (more
                            than the tail's tiles, at most the grid, each share at least 4
                            k-tiles); out: 0 when stream-K is not used */
    int32_t reserved;
    int32_t reserved2;
} gemm_config;

/*
 * gemm -- C = A @ B with row-major A (M x K), row-major B (K x N), row-major fp32 C.
 * Exactly gemm_ex(GEMM_OP_N, GEMM_OP_N, ..., cfg = NULL, stream).
 *
 * The operation is the one "Shared memory and tensor cores" sets up in section
 * 13.1 (C = A @ B for a square problem, whose DRAM traffic the block tiling of
 * sections 13.2-13.3 cuts) with the tensor-core contract of section 13.8 and the
 * WMMA template of section 13.9 (16-bit inputs, products exact, sums in fp32,
 * a float C). Arguments: M, N, K >= 0 (elements); A, B, C device pointers owned
 * by the caller; lda, ldb, ldc leading dimensions in elements; dtype a
 * gemm_dtype; stream a hipStream_t (NULL: the default stream). Returns GEMM_OK
 * after enqueueing, or a gemm_status with nothing enqueued.
 */
int gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
         float* C, int64_t ldc, int dtype, void* stream);

/*
 * gemm_ex -- as gemm, with BLAS-style operand flags and an optional forced
 * configuration. opA must be GEMM_OP_N (GEMM_OP_T returns GEMM_ERR_UNSUPPORTED).
 * opB = GEMM_OP_T reads B column-major (B(k,j) = B[j*ldb + k]). cfg = NULL runs
 * the heuristic; otherwise its "in" fields restrict the choice (a request no
 * compiled kernel satisfies returns GEMM_ERR_UNSUPPORTED).
 *
 * The operand layouts follow the learn-cutedsl README, section 2.4 "Layout and
 * Linear indexing": row-major storage has strides (ld, 1), column-major (1, ld),
 * and GEMM libraries commonly take B column-major (B stored row-major but
 * transposed), the NN / NT / TN / TT naming. cfg (host memory, read during the
 * call only, may be NULL) plays the role of the option / Opts a caller of the
 * pages' launch helpers passes to pick a kernel. Errors as for gemm.
 */
int gemm_ex(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
            int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg, void* stream);

/*
 * gemm_plan -- host-only: the configuration gemm_ex would launch for these
 * arguments, without touching any device. a_addr, b_addr, c_addr are the
 * operand addresses (only their alignment is used), num_cus the compute-unit
 * count and arch the device architecture name (e.g. "gfx950"). Applies the same
 * validation as gemm_ex except pointer checks; fills *out on success.
 *
 * This is the launch heuristic in the role of gpu_opt_choice, "GPU architecture
 * and mapping kernels", section 12.9 "Choosing a launch configuration" (and its
 * exercise that asks for a minimum block count that fills the machine): a pure
 * function of the shape, layouts, alignment and device, so it can be tested
 * without a GPU. request (host memory, may be NULL) restricts the choice as
 * gemm_ex's cfg does; out (host memory) receives the launch. Returns
 * GEMM_ERR_NULL_POINTER for out == NULL, else the status gemm_ex would return
 * for these arguments before launching (GEMM_ERR_DEVICE for an arch other than
 * gfx950).
 */
int gemm_plan(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
              int dtype, uintptr_t a_addr, uintptr_t b_addr, uintptr_t c_addr, int num_cus, const char* arch,
              const gemm_config* request, gemm_config* out);

/*
 * gemm_ex_workspace -- gemm_ex with a caller-provided device workspace, which
 * allows split K: the K range is cut into S slices of whole k-tiles that run as
 * separate workgroups (grid y; the register-staged kernels, the one-tile form of
 * the software-pipelined ones and the fp32 direct-copy tiles), each writing its partial product to its own
 * plane of the workspace, and a second kernel adds the planes in slice order into
 * C, applying any epilogue. The sum
 * order is fixed, so results are reproducible call to call (they differ from the
 * unsplit kernel's by rounding). This fills the machine when M x N has few tiles
 * (the "few blocks" case of "GPU architecture and mapping kernels", section 12.9,
 * and its exercise on a minimum block count). The heuristic splits only if the
 * estimate improves and the workspace suffices; cfg->split_k forces a choice.
 * With a workspace the call may instead pack the operands: one extra kernel
 * copies A and B into zero-padded, 16-byte aligned buffers of whole 256 x 256
 * tiles (K padded to a multiple of 64), so unaligned or ragged operands can run
 * on the fastest kernels; C is written only within M x N. Packing needs
 * (Mp*Kp rounded up to 256 bytes + Np*Kp) elements of the input type, Mp, Np
 * = M, N rounded up to 256, Kp = K rounded up to 64; cfg->pack forces a choice.
 * A third use is the stream-K tail of the persistent software-pipelined kernel
 * ("Shared memory and tensor cores", section 13.10, split-K and stream-K): the
 * tiles that leave the persistent grid's last round partly idle are dealt out as
 * equal shares of their k-tiles to cfg->sk_width workgroups; shares that end
 * inside a tile leave fp32 partial sums in the workspace (sk_width * 512 KiB),
 * which a second kernel adds in k order into C, applying any epilogue (so results
 * are reproducible call to call); cfg->stream_k forces a choice.
 * workspace_bytes = 0 (workspace may be NULL) behaves as gemm_ex. Otherwise the
 * workspace must be 16-byte aligned and its whole declared range must not overlap
 * A, B or C (GEMM_ERR_INVALID_VALUE, checked before any launch); its contents
 * are scratch, and calls that share a workspace must be ordered (one stream). A split needs S * M * round_up(N, 4) * 4 bytes (gemm_plan_workspace
 * reports the amount as workspace_bytes).
 */
int gemm_ex_workspace(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      const void* B, int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg,
                      void* workspace, int64_t workspace_bytes, void* stream);

/*
 * gemm_ex_noalloc -- gemm_ex_workspace for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the workspace is a fixed scratch array of
 * GEMM_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until the
 * process ends. The call allocates and frees nothing. Plans, results and errors
 * are those of gemm_ex_workspace with a workspace of that size (split K or
 * packing only when they fit in it); a forced split or packing that needs more
 * returns GEMM_ERR_INVALID_VALUE with a message that says so. Every call on one
 * GPU shares that GPU's array and the array keeps the last call's contents, so
 * calls that overlap in time on one GPU (several streams, or threads without an
 * order between their calls) race and must not be made; calls ordered on one
 * stream are safe.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)

int gemm_ex_noalloc(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, float* C, int64_t ldc, int dtype, const gemm_config* cfg, void* stream);

/*
 * Fused epilogue ("Shared memory and tensor cores", section 13.10: apply a bias,
 * an activation, a residual add or a type cast to the accumulator before the
 * store, saving a kernel and its memory round trip). gemm_ex_epilogue computes
 *     C[i][j] = act(alpha * (A @ B)[i][j] + beta * R[i][j] + bias[j])
 * with the product accumulated in fp32, the epilogue in fp32, and C stored in
 * out_dtype (round to nearest even). R is read only when beta != 0; it has C's
 * element type and leading dimension ldr, and may be C itself (R == C with
 * ldr == ldc: the in-place BLAS form C = alpha A B + beta C); otherwise it must
 * not overlap C. bias (NULL = none) holds N fp32 values and must not overlap C.
 * GEMM_ACT_GELU_TANH is GELU in its tanh form, x/2 (1 + tanh(sqrt(2/pi) (x +
 * 0.044715 x^3))). An identity epilogue (alpha 1, beta 0, no bias, no
 * activation, fp32 C) is the plain store.
 */
typedef enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1, GEMM_ACT_GELU_TANH = 2 } gemm_activation;

typedef struct gemm_epilogue {
    float alpha, beta;
    const void* R;      /* residual (device pointer), element type out_dtype */
    int64_t ldr;        /* leading dimension of R in elements (>= N when beta != 0) */
    const float* bias;  /* NULL or N fp32 values (device pointer) */
    int32_t activation; /* gemm_activation, applied last */
    int32_t out_dtype;  /* GEMM_F32, GEMM_F16 or GEMM_BF16: element type of C and R */
} gemm_epilogue;

/*
 * gemm_ex_epilogue -- gemm_ex_workspace with a fused epilogue; C's element type
 * is epilogue->out_dtype (epilogue = NULL: plain fp32 C). Errors as for
 * gemm_ex_workspace, plus GEMM_ERR_INVALID_VALUE for a bad out_dtype or
 * activation, a short ldr, or overlaps of R or bias with C; GEMM_ERR_NULL_POINTER
 * for a NULL R with beta != 0. Split K applies the epilogue once, to the
 * complete sum; packing applies it in the product kernel.
 */
int gemm_ex_epilogue(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, int dtype, const gemm_epilogue* epilogue,
                     const gemm_config* cfg, void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_plan_workspace -- host-only: the configuration gemm_ex_epilogue (or, with
 * epilogue = NULL, gemm_ex_workspace) would use with workspace_bytes of workspace
 * (gemm_plan is this with 0 and NULL). */
int gemm_plan_workspace(int opA, int opB, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                        int dtype, uintptr_t a_addr, uintptr_t b_addr, uintptr_t c_addr, int num_cus,
                        const char* arch, int64_t workspace_bytes, const gemm_epilogue* epilogue,
                        const gemm_config* request, gemm_config* out);

/*
 * Grouped and batched products: several independent C = A @ B in one launch
 * ("Grouped Tile Scheduler", learn-cutedsl README section 8.4: the tiles of all
 * problems form one linear index space that a persistent grid walks, each
 * workgroup mapping a linear tile back to its problem by searching the problems'
 * tile offsets; section 8.1's static persistent scheduler strides every
 * workgroup through that space by the grid size).
 *
 * One gemm_problem entry describes `batch` problems of one shape: problem b
 * (0 <= b < batch) reads A + b*stride_a, B + b*stride_b and writes
 * C + b*stride_c (strides in ELEMENTS of the operand's type, >= 0). A single
 * problem is batch = 1 (strides ignored). Every problem follows the conventions
 * above (row-major A, opB for B, fp32 C overwritten, degenerate shapes, the same
 * leading-dimension rules, plus ldc < 2^31); dtype, opA and opB are common to all.
 */
typedef struct gemm_problem {
    int64_t M, N, K;
    const void* A;
    int64_t lda, stride_a;
    const void* B;
    int64_t ldb, stride_b;
    float* C;
    int64_t ldc, stride_c;
    int64_t batch; /* problems in this entry (0 = none) */
} gemm_problem;

/*
 * gemm_grouped -- every problem of problems[0..count) in one kernel launch (more
 * than 16 entries with work are split over several launches on `stream`, in
 * order). problems is a HOST array read during the call only; the operand
 * pointers in it are device pointers. Outputs must not overlap each other or any
 * input (checked over each entry's whole address range, batch included:
 * GEMM_ERR_INVALID_VALUE); within an entry with batch > 1, stride_c must be at
 * least (M-1)*ldc + N. count == 0, or entries without output elements, are
 * no-ops. Only the register-staged configurations (schedule 1) run grouped; cfg
 * restricts the choice as for gemm_ex, and cfg->max_grid caps the persistent grid.
 * Errors as for gemm_ex: everything is validated before the first launch.
 */
int gemm_grouped(int opA, int opB, int dtype, const gemm_problem* problems, int count, const gemm_config* cfg,
                 void* stream);

/* gemm_grouped_plan -- host-only: the configuration gemm_grouped would use (the
 * operand pointers of `problems` are used for their alignment only). */
int gemm_grouped_plan(int opA, int opB, int dtype, const gemm_problem* problems, int count, int num_cus,
                      const char* arch, const gemm_config* request, gemm_config* out);

/* gemm_strided_batched -- gemm_grouped of one entry: `batch` problems of one
 * shape at fixed element strides. */
int gemm_strided_batched(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b, float* C, int64_t ldc,
                         int64_t stride_c, int64_t batch, int dtype, const gemm_config* cfg, void* stream);

/* Number of compiled kernel configurations, and entry i of that menu (GEMM_OK, or
 * GEMM_ERR_INVALID_VALUE for an index out of range). Host-only. */
int gemm_menu_size(void);
int gemm_menu_entry(int index, int* variant, int* dtype, int* opb, gemm_config* out);

/* Compute-unit count and architecture name (NUL-terminated, truncated to len)
 * of HIP device `device`. Returns GEMM_ERR_DEVICE if it cannot be queried. */
int gemm_device_info(int device, int* num_cus, char* arch, int len);

/*
 * Status reporting in the manner of the pages' GPU runtime, "GPU architecture
 * and mapping kernels", section 12.11 "Running on a real GPU: cuda.py": every
 * runtime status is checked and a nonzero one is turned into an error that says
 * what failed; and in the spirit of "Shared memory and tensor cores", section
 * 13.5, where an error is to say what is unsupported and why.
 *
 * gemm_status_string -- a static, NUL-terminated description of a gemm_status
 * value ("unknown gemm_status" for any other int); never NULL, owned by the
 * library, valid for the life of the process.
 */
const char* gemm_status_string(int status);

/* gemm_last_error -- a description of the last failure of a call made on this
 * thread: which argument or runtime call was refused and why ("" after a call
 * that succeeded). The string is thread-local and owned by the library; it stays
 * valid until the next library call on the same thread. */
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_06_AMD_GEMM_H */
