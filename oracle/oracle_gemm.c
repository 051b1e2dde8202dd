/*
 * oracle_gemm.c -- the CPU oracle for the dense matrix product C = A @ B.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the GPU library includes, links or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline use it. It shares no header, table or helper with the GPU path.
 *
 * What it computes (the plain definition, with no blocking or reordering):
 *
 *     Cref[i][j] = sum_{k=0}^{K-1} A(i,k) * B(k,j)        accumulated in double
 *     D[i][j]    = sum_{k=0}^{K-1} |A(i,k)| * |B(k,j)|    the error denominator
 *
 * This is the matrix product that "Shared memory and tensor cores" sets up in
 * section 13.1 (the N = 4096 traffic problem) and that every kernel in that
 * chapter and in "GPU architecture and mapping kernels" (sections 12.8 and 12.11)
 * is checked against. Inputs are decoded exactly to double; every product of two
 * decoded fp32, fp16 or bf16 values is exact in double (at most 48 significant
 * bits), and each addition rounds once in double, in k order. Section 13.8 of the
 * chapter describes the tensor-core contract the GPU path follows: products formed
 * exactly, sums in fp32. The oracle keeps those sums in fp64 instead, so the
 * GPU's fp32 accumulation error is measured against a far more exact value.
 *
 * Operand access (element offsets, leading dimensions in elements):
 *     A(i,k) = A[i*lda + k]        opA = 0 (row-major M x K)
 *     A(i,k) = A[k*lda + i]        opA = 1 (column-major, i.e. row-major K x M)
 *     B(k,j) = B[k*ldb + j]        opB = 0 (row-major K x N)
 *     B(k,j) = B[j*ldb + k]        opB = 1 (column-major, i.e. row-major N x K)
 * dtype: 0 = fp32 (IEEE binary32), 1 = fp16 (IEEE binary16 bit patterns),
 *        2 = bf16 (bfloat16 bit patterns).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double oracle_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double oracle_load(const void* p, int64_t off, int dtype)
{
    if (dtype == 0) return (double)((const float*)p)[off];
    if (dtype == 1) return oracle_decode_f16(((const uint16_t*)p)[off]);
    return oracle_decode_bf16(((const uint16_t*)p)[off]);
}

/* Exposed for the tests: decode one 16-bit pattern. */
double oracle_decode16(uint16_t h, int dtype)
{
    return dtype == 1 ? oracle_decode_f16(h) : oracle_decode_bf16(h);
}

/*
 * oracle_gemm: compute Cref and D for the output rows listed in `rows`
 * (nrows of them; rows == NULL means all M rows in order). Row r of the outputs
 * (Cref and D are nrows x N, row-major, dense) belongs to matrix row rows[r].
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on a bad argument.
 * D may be NULL when the denominator is not wanted.
 */
int oracle_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                const int64_t* rows, int64_t nrows, double* Cref, double* D, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || dtype < 0 || dtype > 2) return -1;
    if (rows == NULL) nrows = M;
    if (nrows == 0 || N == 0) return 0;
    if (K > 0 && (A == NULL || B == NULL)) return -1;
    if (Cref == NULL) return -1;

    /* Decode B once into a dense double array Bd[k][j]. */
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return -1;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j)
                Bd[k * N + j] = oracle_load(B, opB == 0 ? k * ldb + j : j * ldb + k, dtype);
    }

    /* the thread count applies to this call only (a num_threads clause, not the
       process-wide setting, so a later call with nthreads <= 0 gets the default) */
    int nt = 1;
#ifdef _OPENMP
    nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nt;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        double* c = Cref + r * N;
        double* d = D ? D + r * N : NULL;
        if (i < 0 || i >= M) { bad = 1; continue; }
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (d) for (int64_t j = 0; j < N; ++j) d[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_load(A, opA == 0 ? i * lda + k : k * lda + i, dtype);
            const double* b = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
            if (d) {
                double aa = fabs(a);
                for (int64_t j = 0; j < N; ++j) d[j] += aa * fabs(b[j]);
            }
        }
    }
    free(Bd);
    return bad ? -1 : 0;
}

/* Number of threads an OpenMP parallel region of this library would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
