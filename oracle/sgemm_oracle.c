/*
 * CPU oracle for single-precision GEMM — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library. The GPU library never calls it, links it, or shares code
 * with it.
 *
 * What it computes: the plain definition of GEMM given in "From 1% to 94% of
 * cuBLAS, one kernel at a time" (the paragraph defining SGEMM, and the
 * reference semantics of its first, naive kernel): every output element is
 * the length-K dot product of a row of op(A) with a column of op(B), scaled
 * by alpha, plus beta times the old C:
 *
 *     ref[b,i,j] = alpha * sum_{k=0}^{K-1} opA_b[i,k] * opB_b[k,j] + beta * C_b[i,j]
 *     S  [b,i,j] =         sum_{k=0}^{K-1} |opA_b[i,k]| * |opB_b[k,j]|
 *
 * S is the magnitude sum the acceptance bound is scaled by. Everything is
 * accumulated in double precision, k ascending, from the same float32 inputs.
 *
 * Readings where the pages are silent (all stated with the code below):
 *   - op(A)[i,k] = transA ? A[k*lda+i] : A[i*lda+k]  (row-major, cblas style)
 *     op(B)[k,j] = transB ? B[j*ldb+k] : B[k*ldb+j]; batch item b starts at
 *     A + b*strideA, B + b*strideB, C + b*strideC.
 *   - beta == 0: C is not read (a NaN already in C does not propagate).
 *   - alpha == 0 or K == 0: C = beta*C, A and B are not read.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no fused multiply-add, so
 * each product and each sum is one correctly rounded double operation).
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>

typedef long long i64;

struct gemm_args {
    int trans_a, trans_b;
    i64 M, N, K;
    double alpha, beta;
    const float *A; i64 lda, stride_a;
    const float *B; i64 ldb, stride_b;
    const float *C; i64 ldc, stride_c;
    double *ref;    /* [batch][rows][N] of the requested rows */
    double *S;      /* same shape, may be NULL */
    i64 row0, row1; /* rows [row0, row1) of every batch item */
    i64 batch0, batch1;
};

static double op_a(const struct gemm_args *g, const float *A, i64 i, i64 k)
{
    return g->trans_a ? (double)A[k * g->lda + i] : (double)A[i * g->lda + k];
}

static double op_b(const struct gemm_args *g, const float *B, i64 k, i64 j)
{
    return g->trans_b ? (double)B[j * g->ldb + k] : (double)B[k * g->ldb + j];
}

/* One output row: row i of batch item b. acc/sabs are length-N scratch rows.
 * The loop runs k outermost over the row so that every element still sums its
 * K products in ascending k, exactly as the per-element definition does. */
static void one_row(const struct gemm_args *g, i64 b, i64 i, double *acc, double *sabs,
                    double *out_ref, double *out_S)
{
    const float *A = g->A + b * g->stride_a;
    const float *B = g->B + b * g->stride_b;
    const float *C = g->C + b * g->stride_c;
    i64 N = g->N;
    int skip_product = (g->alpha == 0.0 || g->K == 0);

    for (i64 j = 0; j < N; ++j) { acc[j] = 0.0; sabs[j] = 0.0; }
    if (!skip_product) {
        for (i64 k = 0; k < g->K; ++k) {
            double a = op_a(g, A, i, k);
            double abs_a = fabs(a);
            for (i64 j = 0; j < N; ++j) {
                double bkj = op_b(g, B, k, j);
                acc[j] += a * bkj;
                sabs[j] += abs_a * fabs(bkj);
            }
        }
    }
    for (i64 j = 0; j < N; ++j) {
        double r = skip_product ? 0.0 : g->alpha * acc[j];
        if (g->beta != 0.0)
            r += g->beta * (double)C[i * g->ldc + j];
        out_ref[j] = r;
        if (out_S)
            out_S[j] = sabs[j];
    }
}

struct worker {
    const struct gemm_args *g;
    i64 first, last; /* flattened (batch, row) work items [first, last) */
};

static void *run_worker(void *p)
{
    struct worker *w = (struct worker *)p;
    const struct gemm_args *g = w->g;
    i64 rows = g->row1 - g->row0;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(g->N > 0 ? g->N : 1));
    double *sabs = (double *)malloc(sizeof(double) * (size_t)(g->N > 0 ? g->N : 1));
    if (!acc || !sabs) { free(acc); free(sabs); return (void *)1; }
    for (i64 t = w->first; t < w->last; ++t) {
        i64 bi = t / rows, r = t % rows;
        i64 b = g->batch0 + bi, i = g->row0 + r;
        i64 out = (bi * rows + r) * g->N;
        one_row(g, b, i, acc, sabs, g->ref + out, g->S ? g->S + out : NULL);
    }
    free(acc);
    free(sabs);
    return NULL;
}

/*
 * Rows [row0,row1) of batch items [batch0,batch1) of the strided-batched GEMM.
 * ref (and S, if not NULL) receive (batch1-batch0)*(row1-row0)*N doubles in
 * row-major order. Work is split over `threads` POSIX threads by whole rows,
 * which does not change any element's summation order.
 * Returns 0 on success, nonzero if a thread could not be started or allocate.
 */
int oracle_sgemm_rows(int trans_a, int trans_b, i64 M, i64 N, i64 K,
                      double alpha, const float *A, i64 lda, i64 stride_a,
                      const float *B, i64 ldb, i64 stride_b,
                      double beta, const float *C, i64 ldc, i64 stride_c,
                      i64 batch0, i64 batch1, i64 row0, i64 row1,
                      double *ref, double *S, int threads)
{
    struct gemm_args g = {trans_a, trans_b, M, N, K, alpha, beta,
                          A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                          ref, S, row0, row1, batch0, batch1};
    i64 items = (batch1 - batch0) * (row1 - row0);
    if (items <= 0 || N <= 0)
        return 0;
    if (threads < 1) threads = 1;
    if (threads > items) threads = (int)items;
    if (threads > 256) threads = 256;

    pthread_t tid[256];
    struct worker w[256];
    int started = 0, rc = 0;
    for (int t = 0; t < threads; ++t) {
        w[t].g = &g;
        w[t].first = items * t / threads;
        w[t].last = items * (t + 1) / threads;
    }
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, run_worker, &w[t]) != 0) { rc = 1; break; }
        started = t;
    }
    if (rc == 0 && run_worker(&w[0]) != NULL) rc = 1;
    for (int t = 1; t <= started; ++t) {
        void *res = NULL;
        pthread_join(tid[t], &res);
        if (res != NULL) rc = 1;
    }
    if (rc != 0) {
        /* run whatever a missing thread would have done on this one */
        return run_worker(&(struct worker){&g, 0, items}) != NULL;
    }
    return 0;
}

/*
 * Individual elements (b[e], i[e], j[e]) for e < count, each the plain dot
 * product of the definition above: used to check a few outputs of a problem
 * too large to recompute whole.
 */
void oracle_sgemm_elements(int trans_a, int trans_b, i64 K,
                           double alpha, const float *A, i64 lda, i64 stride_a,
                           const float *B, i64 ldb, i64 stride_b,
                           double beta, const float *C, i64 ldc, i64 stride_c,
                           i64 count, const i64 *bs, const i64 *is, const i64 *js,
                           double *ref, double *S)
{
    struct gemm_args g = {trans_a, trans_b, 0, 0, K, alpha, beta,
                          A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                          ref, S, 0, 0, 0, 0};
    int skip_product = (alpha == 0.0 || K == 0);
    for (i64 e = 0; e < count; ++e) {
        const float *Ab = A + bs[e] * stride_a;
        const float *Bb = B + bs[e] * stride_b;
        const float *Cb = C + bs[e] * stride_c;
        double dot = 0.0, sabs = 0.0;
        if (!skip_product) {
            for (i64 k = 0; k < K; ++k) {
                double a = op_a(&g, Ab, is[e], k);
                double b = op_b(&g, Bb, k, js[e]);
                dot += a * b;
                sabs += fabs(a) * fabs(b);
            }
        }
        double r = skip_product ? 0.0 : alpha * dot;
        if (beta != 0.0)
            r += beta * (double)Cb[is[e] * ldc + js[e]];
        ref[e] = r;
        if (S)
            S[e] = sabs;
    }
}
