/*
 * Plain CPU oracle for C = A·B  —  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package's smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU product path never calls it, includes
 * nothing from here and shares no code with it.
 *
 * What it follows: page 1 ("[Multi-Core & GPU Programming] CUDA - Matrix
 * Multiplication"), section [Matrix Multiplication], first loop: every
 * P(i,j) is the sum over k of M(i,k)·N(k,j).  In this library the pages'
 * matrices M, N, P are called A, B, C; all are row-major with leading
 * dimensions in elements (page 1, section [Coalescing], which indexes M as
 * M[row*width + k]).
 *
 * Arithmetic: every float32 operand is widened to double.  A product of two
 * float32 values has at most 48 significant bits, so it is exact in double;
 * only the additions round, in k-ascending order for every element.  Rows
 * are shared out across OpenMP threads; each element is still one plain
 * sequential sum, so the thread count never changes a result.
 *
 * Also the transpose of page 2 ("Lec 29 · GPU Architecture (2)"), §1.4:
 * element (i, j) of the input becomes element (j, i) of the output, copied
 * as a 32-bit word (no arithmetic at all).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no -ffast-math), see build.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_NOT_INTEGER (-2)

static int bad_dims(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (lda < (K > 1 ? K : 1)) return 1;
    if (ldb < (N > 1 ? N : 1)) return 1;
    return 0;
}

/*
 * P[r][c] = sum_k A[i0+r][k] * B[k][j0+c] and, when S is not NULL,
 * S[r][c] = sum_k |A[i0+r][k] * B[k][j0+c]|, for the output window rows
 * [i0, i1) and columns [j0, j1).  P and S are (i1-i0)×(j1-j0) row-major with
 * leading dimensions ldp / lds.  Loop order: for each row, for k ascending,
 * for each column -- the textbook sum for every element, visited row by row.
 */
int oracle_gemm_f64_window(int64_t M, int64_t N, int64_t K,
                           const float *A, int64_t lda,
                           const float *B, int64_t ldb,
                           int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                           double *P, int64_t ldp, double *S, int64_t lds)
{
    if (bad_dims(M, N, K, lda, ldb)) return ORACLE_BAD_ARGS;
    if (i0 < 0 || i1 < i0 || i1 > M || j0 < 0 || j1 < j0 || j1 > N) return ORACLE_BAD_ARGS;
    const int64_t w = j1 - j0;
    if (ldp < w || (S && lds < w)) return ORACLE_BAD_ARGS;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = i0; i < i1; ++i) {
        double *p = P + (i - i0) * ldp;
        double *s = S ? S + (i - i0) * lds : NULL;
        for (int64_t c = 0; c < w; ++c) {
            p[c] = 0.0;
            if (s) s[c] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *brow = B + k * ldb + j0;
            for (int64_t c = 0; c < w; ++c) {
                const double t = a * (double)brow[c];
                p[c] += t;
                if (s) s[c] += fabs(t);
            }
        }
    }
    return ORACLE_OK;
}

/* The whole product: P and S are M×N (the window [0,M)×[0,N)). */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *P, int64_t ldp, double *S, int64_t lds)
{
    return oracle_gemm_f64_window(M, N, K, A, lda, B, ldb, 0, M, 0, N, P, ldp, S, lds);
}

/*
 * A second, independent computation for integer-valued inputs: the same
 * definition in exact 64-bit integer arithmetic, in i-j-k order.  Every
 * operand must be an integer of magnitude below 2^24 (so it is exact in
 * float32); otherwise nothing is written and ORACLE_NOT_INTEGER is returned.
 */
int oracle_gemm_i64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    int64_t *P, int64_t ldp)
{
    if (bad_dims(M, N, K, lda, ldb) || ldp < (N > 1 ? N : 1)) return ORACLE_BAD_ARGS;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) {
            const float v = A[i * lda + k];
            if (!(fabsf(v) < 16777216.0f) || v != truncf(v)) return ORACLE_NOT_INTEGER;
        }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            const float v = B[k * ldb + j];
            if (!(fabsf(v) < 16777216.0f) || v != truncf(v)) return ORACLE_NOT_INTEGER;
        }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];
            P[i * ldp + j] = acc;
        }
    return ORACLE_OK;
}

/*
 * Single-precision model of the pages' kernels, which keep one register
 * accumulator per output and add one product per k step in ascending k
 * (page 1, section [Matrix Multiplication], the "sum" loop, and section
 * [Shared Memory], "Tiled Matrix Multiplication Kernel", the Pvalue loop).
 * Each step is one fused multiply-add rounded once to float32 (C99 fmaf,
 * correctly rounded, round-to-nearest-even), starting from +0.
 */
int oracle_gemm_fma_f32(int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda, const float *B, int64_t ldb,
                        float *C, int64_t ldc)
{
    if (bad_dims(M, N, K, lda, ldb) || ldc < (N > 1 ? N : 1)) return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k)
                acc = fmaf(A[i * lda + k], B[k * ldb + j], acc);
            C[i * ldc + j] = acc;
        }
    return ORACLE_OK;
}

/*
 * Row and column checksums of the product, computed without forming it
 * (Huang-Abraham style), each with the matching sum of absolute products:
 *   row[i]   = sum_k A[i][k] * (sum_j B[k][j])      (= sum_j P[i][j])
 *   rowabs[i]= sum_k |A[i][k]| * (sum_j |B[k][j]|) (= sum_j S[i][j])
 *   col[j]   = sum_k (sum_i A[i][k]) * B[k][j]      (= sum_i P[i][j])
 *   colabs[j]= sum_k (sum_i |A[i][k]|) * |B[k][j]| (= sum_i S[i][j])
 * All in double.  Any output pointer may be NULL.  `work` must hold 4*K
 * doubles.
 */
int oracle_checksums(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     double *row, double *rowabs, double *col, double *colabs,
                     double *work)
{
    if (bad_dims(M, N, K, lda, ldb)) return ORACLE_BAD_ARGS;
    double *bsum = work, *babs = work + K, *asum = work + 2 * K, *aabs = work + 3 * K;
    for (int64_t k = 0; k < K; ++k) {
        double s = 0.0, sa = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            s += (double)B[k * ldb + j];
            sa += fabs((double)B[k * ldb + j]);
        }
        bsum[k] = s;
        babs[k] = sa;
        s = 0.0;
        sa = 0.0;
        for (int64_t i = 0; i < M; ++i) {
            s += (double)A[i * lda + k];
            sa += fabs((double)A[i * lda + k]);
        }
        asum[k] = s;
        aabs[k] = sa;
    }
    for (int64_t i = 0; i < M; ++i) {
        double r = 0.0, ra = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            r += a * bsum[k];
            ra += fabs(a) * babs[k];
        }
        if (row) row[i] = r;
        if (rowabs) rowabs[i] = ra;
    }
    for (int64_t j = 0; j < N; ++j) {
        double c = 0.0, ca = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double b = (double)B[k * ldb + j];
            c += asum[k] * b;
            ca += aabs[k] * fabs(b);
        }
        if (col) col[j] = c;
        if (colabs) colabs[j] = ca;
    }
    return ORACLE_OK;
}

/*
 * Transpose (page 2 §1.4): B(j, i) = A(i, j) for i < M, j < N.  A is M×N
 * with leading dimension lda >= max(1, N), B is N×M with ldb >= max(1, M);
 * both row-major.  Elements are moved as 32-bit words, so every bit pattern
 * (signed zeros, NaN payloads, subnormals) arrives unchanged.  Nothing of B
 * outside its N×M elements is written.
 */
int oracle_transpose(int64_t M, int64_t N, const uint32_t *A, int64_t lda, uint32_t *B, int64_t ldb)
{
    if (M < 0 || N < 0 || lda < (N > 1 ? N : 1) || ldb < (M > 1 ? M : 1)) return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) B[j * ldb + i] = A[i * lda + j];
    return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
