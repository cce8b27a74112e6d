/*
 * FP64 CPU oracle for single-precision GEMM, C = A * B.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load or call this
 * library.  It shares no code, header or constant with the GPU library.
 *
 * What it computes (the operation definition of "Beyond Kernel 7: Closing the
 * Gap to cuBLAS on an H100 FP32 GEMM", section "The operation: GEMM and the
 * precision of the comparison"): for an M x K matrix A and a K x N matrix B,
 * each output element is the dot product of row m of A with column n of B,
 *
 *     C[m][n] = sum over k = 0 .. K-1 of A[m][k] * B[k][n],
 *
 * computing AB only (no alpha, no beta).  Inputs are FP32; this oracle forms
 * every product in double precision (a product of two FP32 values is exact in
 * FP64, 24 + 24 <= 53 significand bits) and adds the products in ascending k
 * in double precision.  It also returns, per element, the magnitude sum
 *
 *     S[m][n] = sum over k of |A[m][k] * B[k][n]|,
 *
 * the scale used by the per-element error bound of the GPU result.
 *
 * Storage is row-major with leading dimensions: A[m*lda + k], B[k*ldb + n],
 * C[m*ldc + n], S[m*lds + n].
 *
 * Threads split the rows of C.  Every element is produced by exactly one
 * thread with the same ascending-k summation, so the result does not depend
 * on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off (no fast-math); see oracle/build.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* One element, written as the definition reads: a single dot product. */
void oracle_dot_f64(int K, const float *A_row, const float *B_col, long ldb,
                    double *c_out, double *s_out)
{
    double c = 0.0, s = 0.0;
    for (int k = 0; k < K; ++k) {
        double p = (double)A_row[k] * (double)B_col[(long)k * ldb];
        c += p;
        s += fabs(p);
    }
    *c_out = c;
    *s_out = s;
}

/* Rows [m_begin, m_end) of the product.  For each row the n-loop is the
 * inner loop so that B is read along its rows; the k-loop is still the
 * outer of the two, so each C[m][n] receives its terms in ascending k,
 * exactly as in oracle_dot_f64. */
static void rows_f64(int m_begin, int m_end, int N, int K,
                     const float *A, long lda, const float *B, long ldb,
                     double *C, long ldc, double *S, long lds)
{
    for (int m = m_begin; m < m_end; ++m) {
        double *c_row = C + (long)m * ldc;
        double *s_row = S + (long)m * lds;
        for (int n = 0; n < N; ++n) {
            c_row[n] = 0.0;
            s_row[n] = 0.0;
        }
        for (int k = 0; k < K; ++k) {
            const double a = (double)A[(long)m * lda + k];
            const float *b_row = B + (long)k * ldb;
            for (int n = 0; n < N; ++n) {
                double p = a * (double)b_row[n];
                c_row[n] += p;
                s_row[n] += fabs(p);
            }
        }
    }
}

typedef struct {
    int m_begin, m_end, N, K;
    const float *A; long lda;
    const float *B; long ldb;
    double *C; long ldc;
    double *S; long lds;
} rows_job;

static void *rows_worker(void *arg)
{
    rows_job *j = (rows_job *)arg;
    rows_f64(j->m_begin, j->m_end, j->N, j->K, j->A, j->lda, j->B, j->ldb,
             j->C, j->ldc, j->S, j->lds);
    return NULL;
}

/* Full product.  C and S are M x N double arrays.  nthreads <= 0 means one
 * thread.  Returns 0, or -1 on bad arguments / thread failure. */
int oracle_gemm_f64(int M, int N, int K,
                    const float *A, long lda, const float *B, long ldb,
                    double *C, long ldc, double *S, long lds, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || !C || !S) return -1;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = M > 0 ? M : 1;
    if (nthreads == 1) {
        rows_f64(0, M, N, K, A, lda, B, ldb, C, ldc, S, lds);
        return 0;
    }
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    rows_job *jobs = (rows_job *)calloc((size_t)nthreads, sizeof(rows_job));
    if (!tid || !jobs) { free(tid); free(jobs); return -1; }
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        rows_job *j = &jobs[t];
        j->m_begin = (int)((long)M * t / nthreads);
        j->m_end = (int)((long)M * (t + 1) / nthreads);
        j->N = N; j->K = K;
        j->A = A; j->lda = lda; j->B = B; j->ldb = ldb;
        j->C = C; j->ldc = ldc; j->S = S; j->lds = lds;
        if (pthread_create(&tid[t], NULL, rows_worker, j) != 0) { rc = -1; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
    return rc;
}

/* Selected elements only: for each i, C[rows[i]][cols[i]] and its S, each by
 * one dot product (oracle_dot_f64).  Used to check large products at sampled
 * positions.  Returns 0, or -1 on bad arguments. */
int oracle_gemm_points_f64(int M, int N, int K,
                           const float *A, long lda, const float *B, long ldb,
                           long npts, const int64_t *rows, const int64_t *cols,
                           double *c_out, double *s_out)
{
    if (npts < 0 || (npts > 0 && (!rows || !cols || !c_out || !s_out))) return -1;
    for (long i = 0; i < npts; ++i) {
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -1;
    }
    for (long i = 0; i < npts; ++i) {
        oracle_dot_f64(K, A + rows[i] * lda, B + cols[i], ldb, &c_out[i], &s_out[i]);
    }
    return 0;
}
