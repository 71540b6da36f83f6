/*
 * CPU oracle for the tiled GEMM  C = A x B  (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path (libtgemm and its
 * Python binding) never calls it, and this file shares no code, header,
 * table or helper with that path.
 *
 * What it computes is the plain definition of the product, as stated in
 * "4.1 CUDA GEMM算子性能优化" (CUDA GEMM operator optimisation), section 1.1:
 * A is M x K, B is K x N, C is M x N and
 *
 *     C[i][j] = sum_{k < K} A[i][k] * B[k][j].
 *
 * The element indexing is the row-major indexing of that page's naive kernel
 * (section 3.1): A[i*lda + k], B[k*ldb + j]; with lda = K, ldb = N this is
 * exactly the page's A[row*K + k], B[k*N + col].  The pipelining described in
 * the "流水化 GPU 内核" (pipelining GPU kernels) skill, Step 5, and in the
 * SM80 ablation plan, section 1.3, only reorders loads and never changes the
 * arithmetic, so the plain definition is the oracle for every variant.
 *
 * Precision: products of two bf16 values (8-bit significands) or two fp32
 * values (24-bit significands) are exact in fp64 (53 bits), so each term is
 * exact and only the fp64 summation rounds (relative error below
 * (K-1) * 2^-53 of the companion sum S below).  int8 products are summed
 * exactly in int64.
 *
 * Besides C the float oracles return the companion S[i][j] = sum_k |A[i][k] *
 * B[k][j]|, the scale against which the per-element tolerances are stated.
 *
 * Loop order is i (rows, spread over OpenMP threads), then k, then j, with
 * a row accumulator per i: the obvious triple loop with no blocking.
 *
 * Every function returns 0 on success and -1 on invalid sizes.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32: widening is a 16-bit shift of
 * the raw bits (exact).  */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bad_sizes(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (lda < (K > 0 ? K : 1) && M > 0 && K > 0) return 1;
    if (ldb < (N > 0 ? N : 1) && K > 0 && N > 0) return 1;
    if (ldc < (N > 0 ? N : 1) && M > 0 && N > 0) return 1;
    return 0;
}

/* fp32 x fp32 -> fp64 reference with companion sum of |products|. */
int oracle_gemm_f32(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, double *S, int64_t ldc)
{
    if (bad_sizes(M, N, K, lda, ldb, ldc)) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        double *s = S + i * ldc;
        for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; s[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)A[i * lda + k];
            const float *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                double p = a * (double)b[j];
                c[j] += p;
                s[j] += fabs(p);
            }
        }
    }
    return 0;
}

/* bf16 x bf16 -> fp64 reference; A and B are raw bf16 bit patterns. */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                     double *C, double *S, int64_t ldc)
{
    if (bad_sizes(M, N, K, lda, ldb, ldc)) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        double *s = S + i * ldc;
        for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; s[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            double a = bf16_bits_to_double(A[i * lda + k]);
            const uint16_t *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                double p = a * bf16_bits_to_double(b[j]);
                c[j] += p;
                s[j] += fabs(p);
            }
        }
    }
    return 0;
}

/* int8 x int8 -> exact int64 reference. */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                   int64_t *C, int64_t ldc)
{
    if (bad_sizes(M, N, K, lda, ldb, ldc)) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        int64_t *c = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) c[j] = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = (int64_t)A[i * lda + k];
            const int8_t *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) c[j] += a * (int64_t)b[j];
        }
    }
    return 0;
}

/*
 * fp32 "one fused multiply-add chain per output" reference:
 *     acc = 0;  for k = 0 .. K-1:  acc = fma(A[i][k], B[k][j], acc)
 * in single precision, k increasing.  This is the per-thread loop of the
 * naive kernel in section 3.1 of the GEMM page with the multiply-add fused,
 * and the order every register-tiled fp32 kernel keeps when it never splits K
 * (sections 5.2 and 9.2 of the same page accumulate each C element in k
 * order).  It is used to check such kernels bit for bit.
 */
int oracle_gemm_f32_fma_chain(int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda, const float *B, int64_t ldb,
                              float *C, int64_t ldc)
{
    if (bad_sizes(M, N, K, lda, ldb, ldc)) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        float *c = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = A[i * lda + k];
            const float *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) c[j] = fmaf(a, b[j], c[j]);
        }
    }
    return 0;
}

/*
 * Sampled variants: the same definitions evaluated only at the listed
 * (row, col) positions, one dot product per position, so that a full-size
 * problem can be checked at a few thousand outputs.  Positions are given as
 * two int64 arrays of length P; outputs are dense arrays of length P.
 */
int oracle_gemm_f32_sampled(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda, const float *B, int64_t ldb,
                            int64_t P, const int64_t *rows, const int64_t *cols,
                            double *C, double *S)
{
    if (bad_sizes(M, N, K, lda, ldb, N > 0 ? N : 1)) return -1;
    int64_t p;
    for (p = 0; p < P; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int64_t i = rows[p], j = cols[p];
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double q = (double)A[i * lda + k] * (double)B[k * ldb + j];
            c += q;
            s += fabs(q);
        }
        C[p] = c;
        S[p] = s;
    }
    return 0;
}

int oracle_gemm_bf16_sampled(int64_t M, int64_t N, int64_t K,
                             const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                             int64_t P, const int64_t *rows, const int64_t *cols,
                             double *C, double *S)
{
    if (bad_sizes(M, N, K, lda, ldb, N > 0 ? N : 1)) return -1;
    int64_t p;
    for (p = 0; p < P; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int64_t i = rows[p], j = cols[p];
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double q = bf16_bits_to_double(A[i * lda + k]) *
                       bf16_bits_to_double(B[k * ldb + j]);
            c += q;
            s += fabs(q);
        }
        C[p] = c;
        S[p] = s;
    }
    return 0;
}

int oracle_gemm_i8_sampled(int64_t M, int64_t N, int64_t K,
                           const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                           int64_t P, const int64_t *rows, const int64_t *cols,
                           int64_t *C)
{
    if (bad_sizes(M, N, K, lda, ldb, N > 0 ? N : 1)) return -1;
    int64_t p;
    for (p = 0; p < P; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int64_t i = rows[p], j = cols[p];
        int64_t c = 0;
        for (int64_t k = 0; k < K; ++k)
            c += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];
        C[p] = c;
    }
    return 0;
}

int oracle_gemm_f32_fma_chain_sampled(int64_t M, int64_t N, int64_t K,
                                      const float *A, int64_t lda,
                                      const float *B, int64_t ldb,
                                      int64_t P, const int64_t *rows,
                                      const int64_t *cols, float *C)
{
    if (bad_sizes(M, N, K, lda, ldb, N > 0 ? N : 1)) return -1;
    int64_t p;
    for (p = 0; p < P; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int64_t i = rows[p], j = cols[p];
        float c = 0.0f;
        for (int64_t k = 0; k < K; ++k) c = fmaf(A[i * lda + k], B[k * ldb + j], c);
        C[p] = c;
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
