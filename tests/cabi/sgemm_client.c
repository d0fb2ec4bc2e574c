/*
 * A plain C caller of libsgemm: test infrastructure for the C ABI.
 *
 * It uses nothing but include/sgemm.h and the HIP runtime's C API: no Python,
 * no PyTorch. It reads one case (operation arguments and the float32 contents
 * of A, B and C) from a file, allocates device memory with hipMalloc, copies
 * the operands in, makes one library call on a stream it creates, copies C
 * back and writes it to a file together with the call's status. The test that
 * drives it compares that C with the CPU oracle and with the same call made
 * through the Python binding.
 *
 * Case file (native byte order):
 *   int64  trans_a, trans_b, M, N, K, lda, ldb, ldc, batch,
 *          stride_a, stride_b, stride_c, entry
 *   double alpha, beta
 *   int64  nA, nB, nC           element counts of the three buffers
 *   float  A[nA], B[nB], C[nC]
 * entry: 0 sgemm, 1 sgemm_strided_batched, 2 sgemm_strided_batched_ws with the
 * workspace sgemm_workspace_size asks for, 3 sgemm_batched with device arrays
 * of item pointers at the given strides, 4 sgemm_colmajor.
 *
 * Output file: int64 status, then float C[nC] (C as the call left it).
 *
 * Invoked as `sgemm_client --errors`, it makes calls whose arguments the
 * library must reject, prints each status with its message, and exits 0 only
 * if every status is the expected negative value.
 *
 * Exit status: 0 when the case ran (whatever the library returned: the status
 * is in the output file), 2 for a usage or file error, 3 for a HIP runtime
 * error outside the library call.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sgemm.h"

#define HIP_OK(expr)                                                                  \
    do {                                                                              \
        hipError_t e_ = (expr);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "sgemm_client: %s: %s\n", #expr, hipGetErrorString(e_)); \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

enum { H_TA, H_TB, H_M, H_N, H_K, H_LDA, H_LDB, H_LDC, H_BATCH, H_SA, H_SB, H_SC, H_ENTRY,
       H_COUNT };

static void read_exact(FILE *f, void *dst, size_t bytes, const char *what)
{
    if (bytes && fread(dst, 1, bytes, f) != bytes) {
        fprintf(stderr, "sgemm_client: short read of %s\n", what);
        exit(2);
    }
}

static float *to_device(const float *h, int64_t n)
{
    float *d = NULL;
    HIP_OK(hipMalloc((void **)&d, (size_t)(n > 0 ? n : 1) * sizeof(float)));
    if (n > 0) HIP_OK(hipMemcpy(d, h, (size_t)n * sizeof(float), hipMemcpyHostToDevice));
    return d;
}

/* Calls the library must refuse before any device work; each returns the
 * negative status of the first bad argument. No buffer is dereferenced. */
static int check_errors(void)
{
    float dummy[16] = {0};
    struct { const char *what; int got; int want; } c[4];
    int n = 0;
    c[n].what = "M < 0";
    c[n].got = sgemm(0, 0, -1, 4, 4, 1.0f, dummy, 4, dummy, 4, 0.0f, dummy, 4, NULL);
    c[n++].want = -3;
    c[n].what = "lda < K (A not transposed)";
    c[n].got = sgemm(0, 0, 4, 4, 8, 1.0f, dummy, 4, dummy, 4, 0.0f, dummy, 4, NULL);
    c[n++].want = -8;
    c[n].what = "C is NULL";
    c[n].got = sgemm(0, 0, 4, 4, 4, 1.0f, dummy, 4, dummy, 4, 0.0f, NULL, 4, NULL);
    c[n++].want = -12;
    c[n].what = "batch < 0";
    c[n].got = sgemm_strided_batched(0, 0, 4, 4, 4, 1.0f, dummy, 4, dummy, 4, 0.0f, dummy, 4,
                                     -1, 16, 16, 16, NULL);
    c[n++].want = -14;
    int ok = 1;
    for (int i = 0; i < n; ++i) {
        printf("%-28s status %d (%s)%s\n", c[i].what, c[i].got, sgemm_status_string(c[i].got),
               c[i].got == c[i].want ? "" : "  <- unexpected");
        ok &= c[i].got == c[i].want;
    }
    return ok ? 0 : 1;
}

int main(int argc, char **argv)
{
    if (argc == 2 && strcmp(argv[1], "--errors") == 0) return check_errors();
    if (argc != 3) {
        fprintf(stderr, "usage: sgemm_client <case file> <output file> | --errors\n");
        return 2;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f) { perror(argv[1]); return 2; }
    int64_t h[H_COUNT], nbuf[3];
    double ab[2];
    read_exact(f, h, sizeof h, "header");
    read_exact(f, ab, sizeof ab, "alpha/beta");
    read_exact(f, nbuf, sizeof nbuf, "buffer lengths");
    for (int i = 0; i < 3; ++i)
        if (nbuf[i] < 0 || nbuf[i] > ((int64_t)1 << 32)) {
            fprintf(stderr, "sgemm_client: bad buffer length %lld\n", (long long)nbuf[i]);
            return 2;
        }
    float *hbuf[3];
    for (int i = 0; i < 3; ++i) {
        hbuf[i] = (float *)malloc((size_t)(nbuf[i] > 0 ? nbuf[i] : 1) * sizeof(float));
        if (!hbuf[i]) { fprintf(stderr, "sgemm_client: out of host memory\n"); return 2; }
        read_exact(f, hbuf[i], (size_t)nbuf[i] * sizeof(float), "operand");
    }
    fclose(f);

    const int ta = (int)h[H_TA], tb = (int)h[H_TB];
    const int M = (int)h[H_M], N = (int)h[H_N], K = (int)h[H_K];
    const int lda = (int)h[H_LDA], ldb = (int)h[H_LDB], ldc = (int)h[H_LDC];
    const int batch = (int)h[H_BATCH];
    const long long sa = h[H_SA], sb = h[H_SB], sc = h[H_SC];
    const float alpha = (float)ab[0], beta = (float)ab[1];

    float *dA = to_device(hbuf[0], nbuf[0]);
    float *dB = to_device(hbuf[1], nbuf[1]);
    float *dC = to_device(hbuf[2], nbuf[2]);
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    int status;
    void *ws = NULL;
    const float **dAarr = NULL, **dBarr = NULL;
    float **dCarr = NULL;
    switch (h[H_ENTRY]) {
    case 0:
        status = sgemm(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, stream);
        break;
    case 1:
        status = sgemm_strided_batched(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc,
                                       batch, sa, sb, sc, stream);
        break;
    case 2: {
        size_t bytes = sgemm_workspace_size(ta, tb, M, N, K, batch);
        if (bytes) HIP_OK(hipMalloc(&ws, bytes));
        status = sgemm_strided_batched_ws(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC,
                                          ldc, batch, sa, sb, sc, ws, bytes, stream);
        break;
    }
    case 3: {
        int nb = batch > 0 ? batch : 1;
        const float **ha = malloc(sizeof(float *) * (size_t)nb);
        const float **hb = malloc(sizeof(float *) * (size_t)nb);
        float **hc = malloc(sizeof(float *) * (size_t)nb);
        if (!ha || !hb || !hc) { fprintf(stderr, "sgemm_client: out of host memory\n"); return 2; }
        for (int i = 0; i < batch; ++i) {
            ha[i] = dA + (long long)i * sa;
            hb[i] = dB + (long long)i * sb;
            hc[i] = dC + (long long)i * sc;
        }
        HIP_OK(hipMalloc((void **)&dAarr, sizeof(float *) * (size_t)nb));
        HIP_OK(hipMalloc((void **)&dBarr, sizeof(float *) * (size_t)nb));
        HIP_OK(hipMalloc((void **)&dCarr, sizeof(float *) * (size_t)nb));
        HIP_OK(hipMemcpy(dAarr, ha, sizeof(float *) * (size_t)nb, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dBarr, hb, sizeof(float *) * (size_t)nb, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dCarr, hc, sizeof(float *) * (size_t)nb, hipMemcpyHostToDevice));
        free(ha); free(hb); free(hc);
        status = sgemm_batched(ta, tb, M, N, K, alpha, dAarr, lda, dBarr, ldb, beta, dCarr, ldc,
                               batch, stream);
        break;
    }
    case 4:
        status = sgemm_colmajor(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, stream);
        break;
    default:
        fprintf(stderr, "sgemm_client: unknown entry %lld\n", (long long)h[H_ENTRY]);
        return 2;
    }
    HIP_OK(hipStreamSynchronize(stream));
    if (nbuf[2] > 0)
        HIP_OK(hipMemcpy(hbuf[2], dC, (size_t)nbuf[2] * sizeof(float), hipMemcpyDeviceToHost));

    FILE *o = fopen(argv[2], "wb");
    if (!o) { perror(argv[2]); return 2; }
    int64_t st64 = status;
    if (fwrite(&st64, sizeof st64, 1, o) != 1 ||
        fwrite(hbuf[2], sizeof(float), (size_t)nbuf[2], o) != (size_t)nbuf[2]) {
        fprintf(stderr, "sgemm_client: write failed\n");
        return 2;
    }
    fclose(o);
    printf("sgemm_client: entry %lld M=%d N=%d K=%d batch=%d status %d (%s)\n",
           (long long)h[H_ENTRY], M, N, K, batch, status, sgemm_status_string(status));

    HIP_OK(hipStreamDestroy(stream));
    if (ws) HIP_OK(hipFree(ws));
    if (dAarr) { HIP_OK(hipFree((void *)dAarr)); HIP_OK(hipFree((void *)dBarr)); HIP_OK(hipFree(dCarr)); }
    HIP_OK(hipFree(dA)); HIP_OK(hipFree(dB)); HIP_OK(hipFree(dC));
    for (int i = 0; i < 3; ++i) free(hbuf[i]);
    return 0;
}
