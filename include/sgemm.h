/*
 * libsgemm — single-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * Computes C = alpha * op(A) @ op(B) + beta * C in fp32, the SGEMM of
 * "From 1% to 94% of cuBLAS, one kernel at a time" (the paragraph defining
 * SGEMM: A is M x K, B is K x N, C is M x N, each output a length-K dot
 * product, row-major storage), with transposed operands expressed as swapped
 * strides as in "Triton Optimization Reference (cuTile -> Triton)", section 2
 * (transpose in pointer arithmetic), and a strided-batched form whose batch
 * index is the second grid axis as in section 3 (grid layout) of that page.
 *
 * Storage (row-major throughout, element strides):
 *   op(A)[i,k] = transA ? A[k*lda + i] : A[i*lda + k]   (A stored K x M or M x K)
 *   op(B)[k,j] = transB ? B[j*ldb + k] : B[k*ldb + j]   (B stored N x K or K x N)
 *   C[i,j]     = C[i*ldc + j]
 *   batch item b uses A + b*strideA, B + b*strideB, C + b*strideC.
 *
 * Ownership: A, B and C are DEVICE pointers owned by the caller; the library
 * keeps no reference after the call returns and allocates no memory (the
 * split-K entry points below use a workspace the caller passes in).
 *
 * Execution: every call is asynchronous on `stream` (a hipStream_t; NULL is
 * the default stream) and never synchronises the host. Results are
 * deterministic: the same call on the same inputs gives the same bits.
 * Calls are thread-safe.
 *
 * Special cases:
 *   - M == 0, N == 0 or batch == 0: nothing is launched.
 *   - alpha == 0 or K == 0: C = beta * C; A and B are not read
 *     (and nothing is launched if beta == 1).
 *   - beta == 0: C is not read, so NaN or Inf already in C never propagates.
 *
 * Accuracy: products and sums are full fp32 (FP32 MFMA, no reduced-precision
 * inputs); each element is within 2e-6 * max(K,1) * (|alpha| * sum_k
 * |op(A)[i,k] op(B)[k,j]| + |beta| |C[i,j]|) of the exact result.
 *
 * Return value (int status):
 *     0  success (the work is queued on the stream);
 *    <0  -(position of the first invalid argument), counted from 1 in the
 *        sgemm_strided_batched argument list: transA -1, transB -2, M -3,
 *        N -4, K -5, A -7, lda -8, B -9, ldb -10, C -12, ldc -13,
 *        batch -14, strideA -15, strideB -16, strideC -17 (negative).
 *        A leading dimension must be at least the stored row length
 *        (lda >= max(1, transA ? M : K), ldb >= max(1, transB ? K : N),
 *        ldc >= max(1, N)); any larger int is accepted. (Most kernels keep
 *        32-bit byte offsets inside a tile; a call with a leading dimension
 *        of 2^21 or more runs a 64-bit-addressed tile instead, see
 *        SGEMM_VARIANT_W64x64.) A NULL pointer is an error only where it
 *        would be dereferenced. Nothing is launched on error.
 *        The variant-forcing entry points return -18 for an unknown variant,
 *        a 4-float variant the operands cannot use, or a variant with 32-bit
 *        in-tile offsets for a leading dimension of 2^21 or more, whatever the
 *        position of their `variant` argument; the split-K entry points
 *        return -19 for an invalid split count, -20 for an invalid
 *        workspace and -21 for a workspace too small for a forced split,
 *        whatever the position of those arguments. Every entry point
 *        returns -22 when one batch item has more output tiles than one
 *        kernel launch holds: more than 2^31 - 1 work-items along the tile
 *        axis (for the 64 x 64 tiles, M x N beyond about 2^34 to 2^35
 *        elements per item, a C of 64 GiB or more). The no-allocation
 *        entry point returns -23 for a split beyond its fixed array, and
 *        sgemm_set_dispatch_overrides -24 / -25 for an invalid table.
 *    >0  a hipError_t raised when querying the device or launching.
 * sgemm_status_string() turns any status into a message.
 *
 * Alignment: none is required. When A and B are 16-byte aligned, lda, ldb,
 * strideA and strideB are multiples of 4, and so is each operand's extent
 * along its stored rows (K for A with transA = 0 and for B with transB = 1,
 * M or N otherwise), the kernels move four floats per load; otherwise a
 * one-float-per-load variant runs.
 */
#ifndef PRECISION_GEMM_AMD_SGEMM_H
#define PRECISION_GEMM_AMD_SGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *sgemm_stream_t; /* hipStream_t; NULL = the default stream */

/* C = alpha * op(A) @ op(B) + beta * C for one matrix triple (batch = 1). */
int sgemm(int transA, int transB, int M, int N, int K,
          float alpha, const float *A, int lda,
                       const float *B, int ldb,
          float beta,        float *C, int ldc,
          sgemm_stream_t stream);

/* The same for `batch` independent triples at element strides strideA,
 * strideB, strideC. strideA or strideB may be 0 (one operand shared by every
 * item); C items must not overlap each other, A or B. */
int sgemm_strided_batched(int transA, int transB, int M, int N, int K,
                          float alpha, const float *A, int lda,
                                       const float *B, int ldb,
                          float beta,        float *C, int ldc,
                          int batch, long long strideA, long long strideB,
                          long long strideC,
                          sgemm_stream_t stream);

/* Message for a status returned by any entry point (static storage). */
const char *sgemm_status_string(int status);

/*
 * Kernel variants the dispatcher chooses among (see sgemm_select_variant).
 * The tile of C one workgroup owns, its waves, and the load width.
 */
enum sgemm_variant {
    SGEMM_VARIANT_AUTO = -1,
    SGEMM_VARIANT_L256x128 = 0, /* 256 x 128 tile, 4 waves, 4-float loads */
    SGEMM_VARIANT_M128x128 = 1, /* 128 x 128 tile, 4 waves, 4-float loads */
    SGEMM_VARIANT_S64x64 = 2,   /*  64 x  64 tile, 4 waves, 4-float loads */
    SGEMM_VARIANT_S64x64_V1 = 3,/*  64 x  64 tile, 4 waves, 1-float loads (any alignment) */
    SGEMM_VARIANT_T64x64 = 4,   /*  64 x  64 tile, 4 waves each on every 4th K-step,
                                    direct-to-LDS streaming (at most one tile per CU over a
                                    deep K, chosen where a long operand over 128 MiB is
                                    contiguous in k and the short one is not) */
    SGEMM_VARIANT_L256x256 = 5, /* 256 x 256 tile, 8 waves (two per SIMD in one workgroup) */
    SGEMM_VARIANT_S64x64_K2 = 6,/*  64 x  64 tile, 8 waves: two groups of 4 split each
                                    32-deep K-step, partial tiles added in LDS */
    SGEMM_VARIANT_M128x128_DMA = 7,/* 128 x 128 tile, 4 waves, direct-to-LDS loads into a
                                      3-stage LDS ring */
    SGEMM_VARIANT_T32x64 = 8,   /*  32 x  64 tile, 8 waves (two per SIMD) each on every 8th
                                    K-step, direct-to-LDS streaming (grids of at most one
                                    such tile per CU over K < 512, or M <= 32) */
    SGEMM_VARIANT_T64x32 = 9,   /*  64 x  32 tile, the same kernel (grids of at most one
                                    such tile per CU over K >= 512, N <= 32, or a last
                                    round of tiles it fills better) */
    SGEMM_VARIANT_GEMV = 10,    /*  matrix-vector kernels without MFMA: N == 1 with
                                    transB == 1, or M == 1 with transA == 0 (the vector
                                    contiguous in k), the matrix either way; or a few
                                    vectors, 2 <= N <= 8, with transA == 0 (B either
                                    way), or a few rows, 2 <= M <= 8, with transB == 1
                                    (A either way); -18 for any other call */
    SGEMM_VARIANT_W64x64 = 11,  /*  64 x  64 tile, 4 waves, 4-float loads, 64-bit addressing
                                    with per-lane predicates instead of 32-bit buffer
                                    offsets: any leading dimension (chosen for calls with
                                    an ld of 2^21 or more) */
    SGEMM_VARIANT_W64x64_V1 = 12,/* the same with 1-float loads (any alignment) */
    SGEMM_VARIANT_P128x128 = 13,/* persistent: one 12-wave workgroup per compute unit, three
                                    groups of 4 waves each on 128 x 128 tiles; the unit's
                                    n = 3q + 1 tiles go q whole to each group and the last
                                    one split over K into thirds, summed in LDS. Needs the
                                    tiles (times batch) to split evenly over the compute
                                    units with n % 3 != 2, and K >= 192 when n % 3 == 1;
                                    strided calls only, no split-K (-18 / -19 otherwise) */
    SGEMM_VARIANT_P64x64 = 14,  /*  the same on 64 x 64 tiles */
    SGEMM_VARIANT_COUNT = 15
};

/*
 * Host-side dispatch decision, exposed for tests and tuning (no device call):
 * the variant sgemm_strided_batched would launch for this shape, given
 * whether the 4-float load path is allowed (`vec4_ok`, see Alignment above)
 * and the device's compute-unit count. Returns an sgemm_variant, or a
 * negative status for invalid dimensions. The flags are those of the call
 * after one normalization the entry points make first: a vector operand whose
 * k elements are adjacent is described contiguous in k (op(B) with N == 1,
 * transB == 0 and ldb == 1 as transB == 1, ldb == K; op(A) with M == 1,
 * transA == 1 and lda == 1 as transA == 0, lda == K; for K > 1), which
 * names the same memory. The leading dimensions are not among the arguments:
 * a call with one of 2^21 or more runs SGEMM_VARIANT_W64x64 (or its 1-float
 * form) in place of any tile or streaming variant returned here. An installed
 * dispatch override for the shape (sgemm_set_dispatch_overrides) comes first.
 */
int sgemm_select_variant(int transA, int transB, int M, int N, int K, int batch,
                         int vec4_ok, int num_cus);

/*
 * Per-shape dispatch overrides: the table an offline tuning sweep produces.
 * "From 1% to 94% of cuBLAS, one kernel at a time" times every configuration
 * that survives its resource filters and finds the best one differs from GPU
 * to GPU (its autotuning step, "What 'sensible' means"); "Triton Optimization
 * Reference (cuTile -> Triton)", section 4 (autotune breadth, per-GPU
 * configuration lists), asks for a tuned choice per backend and GPU. Each
 * record names one call shape and the variant the automatic choice takes for
 * exactly that shape, in place of the cost model's: `entries` holds `count`
 * records of seven ints {transA, transB, M, N, K, batch, variant}, in host
 * memory the library copies (the caller keeps ownership). The shape is the
 * one sgemm_select_variant receives, after its vector normalization; a
 * column-major call is looked up as the row-major product it runs, C^T =
 * op(B)^T op(A)^T (M and N exchanged, transA = the call's transB and
 * transB = its transA). Of two
 * records for one shape the later wins. A call replaces the whole table;
 * count 0 clears it.
 *
 * A record may name any tile or streaming variant (all but SGEMM_VARIANT_GEMV
 * and the persistent variants, which run only some shapes). The automatic
 * choice, sgemm_select_variant included, honours a record only where the
 * call's alignment allows the variant's load width; leading dimensions of
 * 2^21 or more still run the 64-bit-addressed tile.
 *
 * Returns 0; -24 if `entries` is NULL with count > 0 or a record is invalid (a
 * transpose flag other than 0 or 1, a negative size, a variant that may not be
 * named); -25 if count < 0 or count > SGEMM_MAX_DISPATCH_OVERRIDES. On error the
 * installed table is unchanged. Thread-safe: a call running concurrently
 * with a replacement sees the old table or the new one. The table is
 * process-wide and serves every device.
 */
#define SGEMM_MAX_DISPATCH_OVERRIDES (1 << 20)
int sgemm_set_dispatch_overrides(const int *entries, int count);

/* Number of shapes in the installed override table (0: none). */
int sgemm_dispatch_override_count(void);

/*
 * sgemm_strided_batched with the kernel variant forced (testing and tuning):
 * `variant` is an sgemm_variant; SGEMM_VARIANT_AUTO behaves exactly like
 * sgemm_strided_batched. A 4-float variant requested for operands that do
 * not meet its alignment, or an unknown variant, returns -18 (the position
 * of `variant`).
 */
int sgemm_strided_batched_variant(int transA, int transB, int M, int N, int K,
                                  float alpha, const float *A, int lda,
                                               const float *B, int ldb,
                                  float beta,        float *C, int ldc,
                                  int batch, long long strideA, long long strideB,
                                  long long strideC, int variant,
                                  sgemm_stream_t stream);

/*
 * Pointer-array batched form: batch item b computes
 *     C_array[b] = alpha * op(A_array[b]) @ op(B_array[b]) + beta * C_array[b]
 * with the row-major storage, leading dimensions and special cases above.
 * This is the general batched layout next to the strided one of "Triton
 * Optimization Reference (cuTile -> Triton)", section 3 (the batch index on
 * the second grid axis): instead of base + b*stride, each batch item's
 * operands come from an array.
 *
 * A_array, B_array and C_array are DEVICE arrays of `batch` DEVICE pointers,
 * all owned by the caller; the kernels read the arrays, the host never does,
 * so the arrays and their items must stay valid until the work completes.
 * Items may repeat in A_array and B_array (shared operands); C items must not
 * overlap each other or any A or B item. Status codes use the positions of
 * this argument list (A_array -7, B_array -9, C_array -12, batch -14); NULL
 * items are not detected. A_array and B_array may be NULL when alpha == 0 or
 * K == 0, C_array when nothing is written.
 *
 * Alignment: none is required. When lda and ldb allow 4-float loads (see
 * Alignment above), the kernels check each item's A and B pointers on the
 * device and compute an item that is not 16-byte aligned with plain 4-byte
 * loads, which is correct but much slower.
 */
int sgemm_batched(int transA, int transB, int M, int N, int K,
                  float alpha, const float *const *A_array, int lda,
                               const float *const *B_array, int ldb,
                  float beta,        float *const *C_array, int ldc,
                  int batch, sgemm_stream_t stream);

/* sgemm_batched with the kernel variant forced, as sgemm_strided_batched_variant. */
int sgemm_batched_variant(int transA, int transB, int M, int N, int K,
                          float alpha, const float *const *A_array, int lda,
                                       const float *const *B_array, int ldb,
                          float beta,        float *const *C_array, int ldc,
                          int batch, int variant, sgemm_stream_t stream);

/*
 * Split-K forms: the same results as sgemm / sgemm_strided_batched, for grids
 * whose output tiles are too few to occupy the GPU (a small M x N over a deep
 * K, e.g. 256 x 256 x 16384, is 16 tiles for 256 compute units). K is cut into
 * S slices: every (tile, slice) workgroup writes its partial tile to the
 * workspace, then a second kernel forms
 *     C = alpha * (partial_0 + partial_1 + ... + partial_{S-1}) + beta * C
 * summing in slice order, so results are deterministic. This is the split-K
 * that "From 1% to 94% of cuBLAS, one kernel at a time" finds in cuBLAS when it
 * compares kernel 10 with cuBLAS at small sizes (a matmul kernel writing
 * per-slice partial sums, then a reduction kernel adding them).
 *
 * workspace: DEVICE memory owned by the caller, 4-byte aligned, of
 * workspace_bytes bytes; the call uses it until the work completes on
 * `stream`, so calls that overlap on one workspace race. S slices of every
 * batch item take S * 4 * M * N * batch bytes. The call picks S itself (the
 * count that minimises the busiest compute unit's share of the work, with
 * slices at least 256 deep and at most 128 of them) and takes no more slices
 * than the workspace holds; with a NULL
 * workspace, workspace_bytes == 0, or a grid that fills the GPU it runs
 * exactly like the unsplit form. Whether and how much it splits changes only
 * the fp32 rounding order, within the accuracy bound above.
 *
 * Status codes as above, plus -20 when workspace_bytes > 0 and workspace is
 * NULL or not 4-byte aligned.
 */
int sgemm_ws(int transA, int transB, int M, int N, int K,
             float alpha, const float *A, int lda,
                          const float *B, int ldb,
             float beta,        float *C, int ldc,
             void *workspace, size_t workspace_bytes,
             sgemm_stream_t stream);

int sgemm_strided_batched_ws(int transA, int transB, int M, int N, int K,
                             float alpha, const float *A, int lda,
                                          const float *B, int ldb,
                             float beta,        float *C, int ldc,
                             int batch, long long strideA, long long strideB,
                             long long strideC,
                             void *workspace, size_t workspace_bytes,
                             sgemm_stream_t stream);

/*
 * Bytes of workspace with which sgemm_strided_batched_ws (or sgemm_ws, with
 * batch = 1) never takes fewer slices than it would like, on the current
 * device; 0 when it would not split, for invalid arguments, or when no device
 * can be queried. The automatic split depends on the device's compute-unit
 * count, so query on the device that will run the call.
 */
size_t sgemm_workspace_size(int transA, int transB, int M, int N, int K, int batch);

/*
 * sgemm_strided_batched_ws with the variant (as sgemm_strided_batched_variant)
 * and the split count forced (testing and tuning). splits: 0 = the automatic
 * choice, 1 = no split, S >= 2 = slices of round_up(ceil(K / S), BK) k each
 * (BK: the variant's K-step, 16 or 32; the last slice takes the rest, so
 * fewer than S slices can result). A forced split needs its full workspace
 * (-21 otherwise) and a tile variant (-19 for the streaming variants
 * SGEMM_VARIANT_T64x64, SGEMM_VARIANT_T32x64 and SGEMM_VARIANT_T64x32, which
 * split K across their own waves instead, and for SGEMM_VARIANT_GEMV).
 */
int sgemm_strided_batched_ws_variant(int transA, int transB, int M, int N, int K,
                                     float alpha, const float *A, int lda,
                                                  const float *B, int ldb,
                                     float beta,        float *C, int ldc,
                                     int batch, long long strideA, long long strideB,
                                     long long strideC, int variant, int splits,
                                     void *workspace, size_t workspace_bytes,
                                     sgemm_stream_t stream);

/*
 * Host-side split decision of the split-K forms for a given variant, exposed
 * for tests and tuning (no device call): the number of K slices (1 = none)
 * for this shape on `num_cus` compute units with an unlimited workspace, or a
 * negative status (-18 for an unknown variant).
 */
int sgemm_select_splits(int transA, int transB, int M, int N, int K, int batch,
                        int variant, int num_cus);

/*
 * Column-major (BLAS convention) forms of sgemm and sgemm_strided_batched:
 * the same C = alpha * op(A) @ op(B) + beta * C, with
 *   op(A)[i,k] = transA ? A[i*lda + k] : A[k*lda + i]   (A stored M x K or K x M, by columns)
 *   op(B)[k,j] = transB ? B[k*ldb + j] : B[j*ldb + k]
 *   C[i,j]     = C[j*ldc + i]
 * and lda >= max(1, transA ? K : M), ldb >= max(1, transB ? N : K),
 * ldc >= max(1, M). Read by rows, a column-major matrix is
 * its transpose, so the call runs the row-major kernels on
 * C^T = op(B)^T @ op(A)^T with the operands swapped: no data moves and the
 * results are those of the row-major call on the transposed problem.
 * Status codes, special cases, ownership and accuracy are those of the
 * row-major forms, positions counted in this argument list.
 */
int sgemm_colmajor(int transA, int transB, int M, int N, int K,
                   float alpha, const float *A, int lda,
                                const float *B, int ldb,
                   float beta,        float *C, int ldc,
                   sgemm_stream_t stream);

int sgemm_colmajor_strided_batched(int transA, int transB, int M, int N, int K,
                                   float alpha, const float *A, int lda,
                                                const float *B, int ldb,
                                   float beta,        float *C, int ldc,
                                   int batch, long long strideA, long long strideB,
                                   long long strideC,
                                   sgemm_stream_t stream);

/*
 * sgemm_strided_batched_ws_variant's automatic-variant call that allocates
 * nothing and takes no workspace: for callers that cannot call hipMalloc
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The split-K partial tiles go to a fixed array of
 * SGEMM_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * every GPU it runs on until the process ends (hipGetSymbolAddress finds its
 * address once per device, on the first call made with that device
 * current). splits: 0 = the automatic split, with no more slices than the
 * array holds; 1 = no split; S >= 2 = forced as in
 * sgemm_strided_batched_ws_variant, refused with -23 when S slices of
 * 4 * M * N * batch bytes exceed the array (nothing is launched then).
 * Results are bit for bit those of sgemm_strided_batched_ws_variant with
 * SGEMM_VARIANT_AUTO, the same split count and a workspace of
 * SGEMM_NOALLOC_SCRATCH_BYTES. The caller still owns and passes A, B and C.
 * All calls on one GPU share its array and nothing in it is cleared or needs
 * to be: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller. Status codes as
 * sgemm_strided_batched_ws_variant, plus -19 for a split count below 0 or
 * over 65535 and -23 as above.
 */
#define SGEMM_NOALLOC_SCRATCH_BYTES (32u << 20)

int sgemm_strided_batched_noalloc(int transA, int transB, int M, int N, int K,
                                  float alpha, const float *A, int lda,
                                               const float *B, int ldb,
                                  float beta,        float *C, int ldc,
                                  int batch, long long strideA, long long strideB,
                                  long long strideC, int splits,
                                  sgemm_stream_t stream);

/*
 * Host-side check of the buffer-range bookkeeping the tile and streaming
 * kernels use while their load window walks an operand (tests; no device
 * call). A window starts `left_bytes` before the end of the operand and moves
 * `step_bytes` per K-step; ranges[i] receives the range the kernels give the
 * buffer resource of window i: the bytes from its start to the operand's end,
 * at most 2^31 - 1 and at least 0. Returns 0, or -1 for step_bytes <= 0,
 * nsteps < 0 or a NULL `ranges` with nsteps > 0. `ranges` is host memory of
 * nsteps entries owned by the caller.
 */
int sgemm_window_ranges(long long left_bytes, int step_bytes, int nsteps,
                        unsigned int *ranges);

#ifdef __cplusplus
}
#endif

#endif /* PRECISION_GEMM_AMD_SGEMM_H */
