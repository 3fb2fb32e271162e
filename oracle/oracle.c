/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the ternary x int8
 * GEMM and its two backward-style variants.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (cited by page title and section):
 *   [P10425] t27 pull request #10425, "t27c PTX backend: ternary x int8 GEMM
 *            kernel emitted by a .t27 spec (int8 mma.sync), ptx-run glue".
 *   [P10855] t27 pull request #10855, "spec(igla): hslm_bwd_ptx -- HSLM
 *            backward dX and dW as int8 tensor-core PTX written by t27".
 *
 * What is computed (each is a plain definition written out; integer
 * arithmetic is exact, so there is no tolerance and no rounding order):
 *   weight of a 2-bit code c    w = (c & 1) - ((c >> 1) & 1)     [P10425 "What this adds"]
 *   stored W, 4 codes per byte, N-major: code of (k, n) in byte n*(K/4) + k/4,
 *     at bits 2*(k%4) (first code in the low bits -- the reading taken where
 *     the pages do not give the order)                           [P10425 "What this adds"; P10855 PR body]
 *   forward   C[m][n]  = sum_k A[m][k]  * w(k, n)                [P10425 "What this adds"]
 *   dX        dX[m][k] = sum_n dC[m][n] * w(k, n)   (same stored W)   [P10855 PR body, kernel 1]
 *   dW        dW[k][n] = sum_m A[m][k]  * dC[m][n]  (int8 x int8)      [P10855 PR body, kernel 2]
 *
 * Sums are taken in int64.  A sum outside the int32 range is counted as an
 * overflow and stored wrapped to its low 32 bits; every entry point returns the
 * number of such outputs (the "i32 overflow bound" of [P10425 "What this adds"]
 * and the k <= 131071 bound of [P10855 PR body] are the conditions under which
 * this count is zero for every input).
 *
 * Threads split the outer output index only; each output is one serial sum.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

/* ---------------------------------------------------------------------- */
/* the code -> weight rule and the stored layout                          */
/* ---------------------------------------------------------------------- */

static int weight_of_code(unsigned c)
{
    return (int)(c & 1u) - (int)((c >> 1) & 1u);
}

static unsigned code_at(const uint8_t *Wp, int64_t K, int64_t k, int64_t n)
{
    uint8_t byte = Wp[n * (K / 4) + k / 4];
    return (byte >> (2 * (k % 4))) & 3u;
}

int oracle_weight_of_code(int code)
{
    return weight_of_code((unsigned)code & 3u);
}

/* codes[n*K + k] = code of (k, n), for all k < K, n < N */
void oracle_unpack(const uint8_t *Wp, int64_t N, int64_t K, uint8_t *codes)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)code_at(Wp, K, k, n);
}

/* inverse of oracle_unpack: Wp[n*(K/4) + k/4] holds code (k, n) at bits 2*(k%4) */
void oracle_pack(const uint8_t *codes, int64_t N, int64_t K, uint8_t *Wp)
{
    memset(Wp, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Wp[n * (K / 4) + k / 4] |= (uint8_t)((codes[n * K + k] & 3u) << (2 * (k % 4)));
}

/* w[n*K + k] = weight of (k, n) as int8 */
void oracle_decode(const uint8_t *Wp, int64_t N, int64_t K, int8_t *w)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w[n * K + k] = (int8_t)weight_of_code(code_at(Wp, K, k, n));
}

/* ---------------------------------------------------------------------- */
/* helpers: int64 -> int32 with overflow count; a row-split thread pool   */
/* ---------------------------------------------------------------------- */

static int32_t narrow(int64_t s, int64_t *overflows)
{
    if (s < INT32_MIN || s > INT32_MAX)
        ++*overflows;
    return (int32_t)(uint32_t)(uint64_t)s;
}

typedef struct job {
    int op;                 /* 0 fwd, 1 dx, 2 dw */
    const int8_t *X;        /* A (fwd, dw) or dC (dx) */
    const int8_t *Y;        /* decoded w [N][K] (fwd, dx) or dC (dw) */
    int32_t *out;
    int64_t M, N, K;
    int64_t lo, hi;         /* range of the outer output index */
    int64_t overflows;
} job;

/* C[m][n] = sum_k A[m][k] * w[n][k], for m in [lo, hi) */
static void run_fwd(job *j)
{
    const int64_t N = j->N, K = j->K;
    for (int64_t m = j->lo; m < j->hi; ++m) {
        const int8_t *a = j->X + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *w = j->Y + n * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)a[k] * (int64_t)w[k];
            j->out[m * N + n] = narrow(s, &j->overflows);
        }
    }
}

/* dX[m][k] = sum_n dC[m][n] * w[n][k], for m in [lo, hi) */
static void run_dx(job *j)
{
    const int64_t N = j->N, K = j->K;
    int64_t *acc = (int64_t *)malloc((size_t)K * sizeof(int64_t));
    for (int64_t m = j->lo; m < j->hi; ++m) {
        memset(acc, 0, (size_t)K * sizeof(int64_t));
        for (int64_t n = 0; n < N; ++n) {
            const int64_t g = j->X[m * N + n];
            const int8_t *w = j->Y + n * K;
            for (int64_t k = 0; k < K; ++k)
                acc[k] += g * (int64_t)w[k];
        }
        for (int64_t k = 0; k < K; ++k)
            j->out[m * K + k] = narrow(acc[k], &j->overflows);
    }
    free(acc);
}

/* dW[k][n] = sum_m A[m][k] * dC[m][n], for k in [lo, hi) */
static void run_dw(job *j)
{
    const int64_t M = j->M, N = j->N, K = j->K;
    int64_t *acc = (int64_t *)malloc((size_t)N * sizeof(int64_t));
    for (int64_t k = j->lo; k < j->hi; ++k) {
        memset(acc, 0, (size_t)N * sizeof(int64_t));
        for (int64_t m = 0; m < M; ++m) {
            const int64_t a = j->X[m * K + k];
            const int8_t *g = j->Y + m * N;
            for (int64_t n = 0; n < N; ++n)
                acc[n] += a * (int64_t)g[n];
        }
        for (int64_t n = 0; n < N; ++n)
            j->out[k * N + n] = narrow(acc[n], &j->overflows);
    }
    free(acc);
}

static void *run_job(void *p)
{
    job *j = (job *)p;
    if (j->op == 0)
        run_fwd(j);
    else if (j->op == 1)
        run_dx(j);
    else
        run_dw(j);
    return NULL;
}

/* split [0, outer) over `threads` threads; returns the total overflow count */
static int64_t run_split(job proto, int64_t outer, int threads)
{
    if (threads < 1)
        threads = 1;
    if ((int64_t)threads > outer)
        threads = (int)(outer > 0 ? outer : 1);
    job *jobs = (job *)calloc((size_t)threads, sizeof(job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int64_t total = 0;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = proto;
        jobs[t].lo = outer * t / threads;
        jobs[t].hi = outer * (t + 1) / threads;
        jobs[t].overflows = 0;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tid[t], NULL, run_job, &jobs[t]);
    run_job(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tid[t], NULL);
    for (int t = 0; t < threads; ++t)
        total += jobs[t].overflows;
    free(jobs);
    free(tid);
    return total;
}

/* ---------------------------------------------------------------------- */
/* entry points                                                            */
/* ---------------------------------------------------------------------- */

/* C[M][N] = A[M][K] x W[K][N];  A int8 [M][K], Wp uint8 [N][K/4], K % 4 == 0.
 * Returns the number of outputs whose exact value is outside int32, or -1 on
 * bad arguments. */
int64_t oracle_fwd(const int8_t *A, const uint8_t *Wp, int32_t *C,
                   int64_t M, int64_t N, int64_t K, int threads)
{
    if (M < 1 || N < 1 || K < 1 || K % 4)
        return -1;
    int8_t *w = (int8_t *)malloc((size_t)(N * K));
    oracle_decode(Wp, N, K, w);
    job proto = {0, A, w, C, M, N, K, 0, 0, 0};
    int64_t r = run_split(proto, M, threads);
    free(w);
    return r;
}

/* dX[M][K] = dC[M][N] x W^T;  dC int8 [M][N], Wp uint8 [N][K/4] (the forward
 * buffer), K % 4 == 0. */
int64_t oracle_dx(const int8_t *dC, const uint8_t *Wp, int32_t *dX,
                  int64_t M, int64_t N, int64_t K, int threads)
{
    if (M < 1 || N < 1 || K < 1 || K % 4)
        return -1;
    int8_t *w = (int8_t *)malloc((size_t)(N * K));
    oracle_decode(Wp, N, K, w);
    job proto = {1, dC, w, dX, M, N, K, 0, 0, 0};
    int64_t r = run_split(proto, M, threads);
    free(w);
    return r;
}

/* dW[K][N] = A^T x dC;  A int8 [M][K], dC int8 [M][N]. */
int64_t oracle_dw(const int8_t *A, const int8_t *dC, int32_t *dW,
                  int64_t M, int64_t N, int64_t K, int threads)
{
    if (M < 1 || N < 1 || K < 1)
        return -1;
    job proto = {2, A, dC, dW, M, N, K, 0, 0, 0};
    return run_split(proto, K, threads);
}
