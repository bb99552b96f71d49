/*
 * oracle_gemm.c -- the CPU oracle for single-precision GEMM, C = A x B.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU path must
 * compute and is used to check it.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code with
 * the HIP library and the HIP library never calls it.
 *
 * Sources (web pages this project follows):
 *   [GEMM-1024]  "GEMM kernel test code & optimization (1024^3 experiment)",
 *                teach-meaning.tistory.com/1513
 *   [AutoMine2]  "[AutoMine++] #2 matmul trial and error",
 *                velog.io/@levelstage/AutoMinepp2
 *
 * What is computed (plain definition, no blocking, no reordering of a sum):
 *   - C_ij = sum over k = 0..K-1 of A_ik * B_kj.  This is the per-element
 *     definition in [GEMM-1024], section "Mathematical definition".  The
 *     k sum runs strictly in increasing k, as in the CPU triple loop of
 *     [AutoMine2], section "Intuitive implementation (by CPU)".
 *   - Layout is row-major: A[i*lda + k], B[k*ldb + j].  [GEMM-1024],
 *     section "Memory layout", gives lda = K and ldb = N; general leading
 *     dimensions are allowed here.
 *   - Accumulation is in IEEE binary64.  Each product of two binary32
 *     values is exact in binary64 (24 + 24 significand bits <= 53), so the
 *     only rounding is in the running sum.
 *   - The result is also rounded once to binary32 (round to nearest even)
 *     to give C32.
 *   - S_ij = sum over k of |A_ik * B_kj| is returned beside C.  It scales
 *     the tolerance used for floating-point inputs.
 *
 * Threads split the rows of C; each element is summed by one thread in the
 * same k order, so results do not depend on the thread count.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

/* One output element, by the definition: k ascending, binary64 sum. */
static void oracle_entry(int64_t K, const float *A, int64_t lda,
                         const float *B, int64_t ldb, int64_t i, int64_t j,
                         double *c_out, double *s_out)
{
    double acc = 0.0;
    double mag = 0.0;
    const float *a_row = A + i * lda;
    for (int64_t k = 0; k < K; ++k) {
        double p = (double)a_row[k] * (double)B[k * ldb + j];
        acc += p;
        mag += fabs(p);
    }
    *c_out = acc;
    *s_out = mag;
}

typedef struct {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    double *C64;
    float *C32;
    double *S64;
    int64_t ldc;
    int64_t row_begin, row_end;
} full_job;

static void *full_worker(void *arg)
{
    full_job *job = (full_job *)arg;
    for (int64_t i = job->row_begin; i < job->row_end; ++i) {
        for (int64_t j = 0; j < job->N; ++j) {
            double c, s;
            oracle_entry(job->K, job->A, job->lda, job->B, job->ldb, i, j, &c, &s);
            int64_t o = i * job->ldc + j;
            if (job->C64) job->C64[o] = c;
            if (job->C32) job->C32[o] = (float)c;
            if (job->S64) job->S64[o] = s;
        }
    }
    return NULL;
}

#define ORACLE_MAX_THREADS 256

/*
 * Full product.  C64, C32 and S64 are M x N row-major with leading dimension
 * ldc; any of them may be NULL.  Returns 0 on success, -1 on invalid
 * arguments (negative sizes, leading dimension too small, a needed pointer
 * NULL).  Rows of a thread that could not be started are done by the caller.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda, const float *B, int64_t ldb,
                double *C64, float *C32, double *S64, int64_t ldc,
                int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (ldc < N) return -1;
    if (M == 0 || N == 0) return 0;
    if (K > 0 && (A == NULL || B == NULL || lda < K || ldb < N)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > ORACLE_MAX_THREADS) nthreads = ORACLE_MAX_THREADS;
    if (nthreads > M) nthreads = (int)M;

    full_job jobs[ORACLE_MAX_THREADS];
    pthread_t tids[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS] = {0};
    int64_t per = M / nthreads, extra = M % nthreads, row = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t rows = per + (t < extra ? 1 : 0);
        full_job j = {M, N, K, A, lda, B, ldb, C64, C32, S64, ldc, row, row + rows};
        jobs[t] = j;
        row += rows;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tids[t], NULL, full_worker, &jobs[t]) == 0) started[t] = 1;
    full_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(tids[t], NULL);
        else full_worker(&jobs[t]); /* rows of a thread that did not start */
    }
    return 0;
}

typedef struct {
    int64_t K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    const int64_t *rows, *cols;
    double *c64;
    float *c32;
    double *s64;
    int64_t begin, end;
} entries_job;

static void *entries_worker(void *arg)
{
    entries_job *job = (entries_job *)arg;
    for (int64_t e = job->begin; e < job->end; ++e) {
        double c, s;
        oracle_entry(job->K, job->A, job->lda, job->B, job->ldb,
                     job->rows[e], job->cols[e], &c, &s);
        if (job->c64) job->c64[e] = c;
        if (job->c32) job->c32[e] = (float)c;
        if (job->s64) job->s64[e] = s;
    }
    return NULL;
}

/*
 * Selected elements C[rows[e], cols[e]] for e < count, each by the same
 * definition as oracle_gemm (bit-identical to the full product's entry).
 * Returns 0 on success, -1 on invalid arguments (an index out of range
 * included).
 */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda, const float *B, int64_t ldb,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        double *c64, float *c32, double *s64, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (count == 0) return 0;
    if (rows == NULL || cols == NULL) return -1;
    if (K > 0 && (A == NULL || B == NULL || lda < K || ldb < N)) return -1;
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > ORACLE_MAX_THREADS) nthreads = ORACLE_MAX_THREADS;
    if (nthreads > count) nthreads = (int)count;

    entries_job jobs[ORACLE_MAX_THREADS];
    pthread_t tids[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS] = {0};
    int64_t per = count / nthreads, extra = count % nthreads, at = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t n = per + (t < extra ? 1 : 0);
        entries_job j = {K, A, lda, B, ldb, rows, cols, c64, c32, s64, at, at + n};
        jobs[t] = j;
        at += n;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tids[t], NULL, entries_worker, &jobs[t]) == 0) started[t] = 1;
    entries_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(tids[t], NULL);
        else entries_worker(&jobs[t]);
    }
    return 0;
}
