/*
 * FP64 CPU oracle for  D = alpha * A * op(B) + beta * C   (row-major, FP32 storage).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or constant with the HIP library.
 *
 * What it follows:
 *   - "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 1.1:
 *     C(MxN) = A(MxK) x B(KxN); each C[i][j] is K multiply-adds and the outputs
 *     are independent.  Section 2.1 fixes row-major storage: A[row*K+k],
 *     B[k*N+col], C[row*N+col] (leading dimensions lda/ldb/ldc generalise the
 *     row length).
 *   - Baidu Cloud article comparing naive and 2-D block-tiled CUDA matmul, the
 *     paragraph on the naive mapping: the general form D = alpha*A*B^T + beta*C,
 *     where with B transposed C[i][j] is the dot product of row i of A with row j
 *     of B.  Hence op(B)=B^T reads B stored N x K, and element (k,j) of op(B) is
 *     B[j*ldb + k].
 *   - Same article, paragraph on computation logic: every kernel performs the same
 *     m*n*k multiply-adds and reaches the same mathematical result; so the oracle
 *     is that definition written out, accumulated in FP64.
 *
 * Definition computed for every requested row i and every column j < N:
 *     acc  = sum_{k<K} a(i,k) * b(k,j)          (k ascending, FP64)
 *     S    = sum_{k<K} |a(i,k) * b(k,j)|        (the magnitude sum used by the error bound)
 *     D    = alpha*acc + (beta != 0 ? beta*C[i][j] : 0)
 * Each product of two FP32 values is exact in FP64 (24+24 bits <= 53), so the
 * only rounding is in the FP64 sums: at most K*2^-53*S, far below the FP32
 * tolerance the GPU results are held to.
 *
 * Readings where the pages are silent (listed with the design notes):
 *   - beta == 0 means C is not read (NaN/Inf in C do not propagate);
 *   - alpha == 0 or K == 0 gives D = beta*C;
 *   - M == 0 or N == 0 is an empty result.
 *
 * Threading: rows are independent, so they are split across OpenMP threads; each
 * output is still summed by one thread in k-ascending order.
 */
#include <math.h>
#include <stdint.h>
#include <omp.h>

/* element (k, j) of op(B) */
static double opb(const float *B, int64_t ldb, int transB, int64_t k, int64_t j)
{
    return transB ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
}

/* One output row: fills D[0..N) and S[0..N) for row i. */
static void one_row(int64_t N, int64_t K, double alpha,
                    const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                    double beta, const float *C, int64_t ldc,
                    int64_t i, double *D, double *S)
{
    for (int64_t j = 0; j < N; ++j) {
        D[j] = 0.0;
        S[j] = 0.0;
    }
    if (alpha == 0.0) {
        /* the product term vanishes; A and B are not read */
        for (int64_t j = 0; j < N; ++j)
            D[j] = (beta != 0.0) ? beta * (double)C[i * ldc + j] : 0.0;
        return;
    }
    if (transB) {
        /* op(B)(k,j) = B[j][k]: walk row j of B, contiguous in k */
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)A[i * lda + k] * opb(B, ldb, 1, k, j);
                acc += p;
                s += fabs(p);
            }
            D[j] = acc;
            S[j] = s;
        }
    } else {
        /* op(B)(k,j) = B[k][j]: same k-ascending sums, walked row by row of B */
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)A[i * lda + k];
            for (int64_t j = 0; j < N; ++j) {
                double p = a * opb(B, ldb, 0, k, j);
                D[j] += p;
                S[j] += fabs(p);
            }
        }
    }
    for (int64_t j = 0; j < N; ++j) {
        double d = alpha * D[j];
        if (beta != 0.0)
            d += beta * (double)C[i * ldc + j];
        D[j] = d;
    }
}

/*
 * Rows rows[0..nrows) of D and S, written densely: D[r*N + j], S[r*N + j].
 * alpha and beta are the FP32 values the GPU receives, widened to FP64.
 * C may be NULL when beta == 0.  nthreads <= 0 uses the OpenMP default.
 * Returns the number of threads that ran (for reporting), or -1 on bad input.
 */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, float alpha,
                     const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                     float beta, const float *C, int64_t ldc,
                     const int64_t *rows, int64_t nrows,
                     double *D, double *S, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || (transB != 0 && transB != 1))
        return -1;
    if (beta != 0.0f && C == 0 && nrows > 0 && N > 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int used = 1;
    const double da = (double)alpha, db = (double)beta;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t r = 0; r < nrows; ++r) {
        if (r == 0)
            used = omp_get_num_threads();
        one_row(N, K, da, A, lda, B, ldb, transB, db, C, ldc, rows[r], D + r * N, S + r * N);
    }
    return used;
}
