/*
 * Host-side checks of libsgemm under AddressSanitizer: test infrastructure.
 *
 * Built with clang -fsanitize=address and linked to a host-only build of the
 * library that is itself instrumented (no device code: every path exercised
 * here returns before the first HIP call). It drives the host logic over many
 * seeded arguments:
 *   - every status string;
 *   - the dispatch decisions (sgemm_select_variant, sgemm_select_splits) over
 *     random shapes, batches, CU counts and variants, checking their ranges,
 *     with a per-shape override table installed;
 *   - the override table itself (sgemm_set_dispatch_overrides): lookups,
 *     refusal of invalid tables, random replacement and clearing;
 *   - the buffer-window countdown (sgemm_window_ranges) against the bytes
 *     left, for operands of up to 300 GiB;
 *   - argument validation of every entry point, and quick returns, with
 *     pointers that must never be dereferenced.
 * A memory error aborts the run with an AddressSanitizer report; a wrong
 * result is counted and printed. Exit status 0 only if every check passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sgemm.h"

static int failures = 0;

#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            if (failures < 20) {              \
                fprintf(stderr, __VA_ARGS__); \
                fputc('\n', stderr);          \
            }                                 \
            ++failures;                       \
        }                                     \
    } while (0)

/* xorshift64: a fixed, seeded sequence of arguments */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

/* A dimension (at least 1) from a mix of scales: tiny, around the tile
   sizes, large and close to the int range. */
static int dim(void)
{
    switch (next_u64() % 6) {
    case 0: return 1 + (int)(next_u64() % 8);
    case 1: return 1 + (int)(next_u64() % 130);
    case 2: return 1 + (int)(next_u64() % 5000);
    case 3: return 1 + (int)(next_u64() % 70000);
    case 4: return 1 << (next_u64() % 31);
    default: return 1 + (int)(next_u64() % 0x7ffffffeu);
    }
}

static void status_strings(void)
{
    for (int st = -64; st <= 1100; ++st) {
        const char *m = sgemm_status_string(st);
        CHECK(m != NULL && m[0] != '\0', "status %d: no message", st);
    }
    const int extremes[] = {-2147483647 - 1, 2147483647};
    for (int i = 0; i < 2; ++i)
        CHECK(sgemm_status_string(extremes[i]) != NULL, "status %d: no message", extremes[i]);
}

static void dispatch(int rounds)
{
    for (int r = 0; r < rounds; ++r) {
        const int tA = (int)(next_u64() % 2), tB = (int)(next_u64() % 2);
        const int M = dim(), N = dim(), K = dim();
        const int batch = 1 + (int)(next_u64() % 600);
        const int vec4 = (int)(next_u64() % 2), cus = 1 + (int)(next_u64() % 1024);
        const int v = sgemm_select_variant(tA, tB, M, N, K, batch, vec4, cus);
        CHECK(v >= 0 && v < SGEMM_VARIANT_COUNT, "select_variant(%d,%d,%d,%d,%d,%d,%d,%d) = %d",
              tA, tB, M, N, K, batch, vec4, cus, v);
        const int variant = (int)(next_u64() % (SGEMM_VARIANT_COUNT + 2)) - 1;
        const int s = sgemm_select_splits(tA, tB, M, N, K, batch, variant, cus);
        if (variant < 0 || variant >= SGEMM_VARIANT_COUNT)
            CHECK(s == -18, "select_splits with variant %d = %d", variant, s);
        else
            CHECK(s >= 1 && s <= 65535, "select_splits(%d,%d,%d,%d,%d,%d,%d,%d) = %d", tA, tB, M, N,
                  K, batch, variant, cus, s);
    }
    /* invalid arguments of the chooser */
    CHECK(sgemm_select_variant(2, 0, 4, 4, 4, 1, 1, 256) < 0, "transA = 2 accepted");
    CHECK(sgemm_select_variant(0, 0, -1, 4, 4, 1, 1, 256) < 0, "M = -1 accepted");
}

/* Per-shape dispatch overrides: install, look up, refuse invalid tables
   whole, replace and clear, with seeded random tables in between. */
static void overrides(int rounds)
{
    enum { NREC = 64 };
    int rec[7 * NREC];
    for (int i = 0; i < NREC; ++i) {
        int *e = rec + 7 * i;
        e[0] = i & 1;
        e[1] = (i >> 1) & 1;
        e[2] = 64 + i;
        e[3] = 128;
        e[4] = 256;
        e[5] = 1 + i % 3;
        e[6] = i % 2 ? SGEMM_VARIANT_M128x128 : SGEMM_VARIANT_W64x64_V1;
    }
    CHECK(sgemm_set_dispatch_overrides(rec, NREC) == 0, "override table refused");
    CHECK(sgemm_dispatch_override_count() == NREC, "override count");
    for (int i = 0; i < NREC; ++i) {
        const int *e = rec + 7 * i;
        const int v = sgemm_select_variant(e[0], e[1], e[2], e[3], e[4], e[5], 1, 256);
        CHECK(v == e[6], "override %d: %d, want %d", i, v, e[6]);
    }
    rec[7 * 10 + 6] = SGEMM_VARIANT_GEMV;
    CHECK(sgemm_set_dispatch_overrides(rec, NREC) == -24, "GEMV override accepted");
    CHECK(sgemm_dispatch_override_count() == NREC, "refused table changed the installed one");
    CHECK(sgemm_set_dispatch_overrides(NULL, 1) == -24, "NULL entries accepted");
    CHECK(sgemm_set_dispatch_overrides(NULL, -1) == -25, "negative count accepted");
    int *big = (int *)malloc(7 * 4096 * sizeof(int));
    for (int r = 0; r < rounds; ++r) {
        const int n = (int)(next_u64() % 4096);
        int valid = 1;
        for (int i = 0; i < 7 * n; ++i) {
            const int f = i % 7;
            big[i] = f < 2 ? (int)(next_u64() % 2) : f < 6 ? (int)(next_u64() % 3000)
                                                           : (int)(next_u64() % SGEMM_VARIANT_COUNT);
            if (f == 6 && (big[i] == SGEMM_VARIANT_GEMV || big[i] >= SGEMM_VARIANT_P128x128))
                valid = 0;
        }
        if (n > 0 && next_u64() % 8 == 0) {
            big[7 * (n - 1) + 2] = -1; /* a negative size */
            valid = 0;
        }
        const int st = sgemm_set_dispatch_overrides(n ? big : NULL, n);
        CHECK(st == (valid ? 0 : -24), "random table %d: %d", r, st);
    }
    free(big);
    CHECK(sgemm_set_dispatch_overrides(rec, 0) == 0, "clearing refused");
    CHECK(sgemm_dispatch_override_count() == 0, "table not cleared");
}

static void windows(int rounds)
{
    enum { MAXSTEPS = 4096 };
    unsigned int *ranges = (unsigned int *)malloc(MAXSTEPS * sizeof(unsigned int));
    const long long kMax = 2147483647LL;
    const int steps_bytes[] = {16, 64, 128, 256, 1024, 16384, 65536, 1 << 20, 1 << 24};
    for (int r = 0; r < rounds; ++r) {
        const int step = steps_bytes[next_u64() % (sizeof steps_bytes / sizeof steps_bytes[0])];
        /* anywhere up to 300 GiB, or within a few thousand steps of the cap */
        const long long left =
            next_u64() % 2 ? (long long)(next_u64() % (300ULL << 30)) - 4096
                           : kMax + (long long)(next_u64() % 8192) * step - 4096LL * step +
                                 (long long)(next_u64() % 64);
        const int n = 1 + (int)(next_u64() % MAXSTEPS);
        CHECK(sgemm_window_ranges(left, step, n, ranges) == 0, "window_ranges refused");
        for (int i = 0; i < n; ++i) {
            long long want = left - (long long)i * step;
            want = want < 0 ? 0 : want > kMax ? kMax : want;
            if ((long long)ranges[i] != want) {
                CHECK(0, "window %d of %lld bytes, step %d: %u, want %lld", i, left, step,
                      ranges[i], want);
                break;
            }
        }
    }
    CHECK(sgemm_window_ranges(1000, 0, 4, ranges) < 0, "step 0 accepted");
    CHECK(sgemm_window_ranges(1000, 64, 4, NULL) < 0, "NULL ranges accepted");
    CHECK(sgemm_window_ranges(1000, 64, 0, NULL) == 0, "zero steps refused");
    free(ranges);
}

static void arguments(void)
{
    /* Addresses that must never be dereferenced: validation and quick
       returns happen before any memory access or HIP call. */
    float *const P = (float *)(uintptr_t)4096;
    const float *const *const PA = (const float *const *)(uintptr_t)8192;
    float *const *const PC = (float *const *)(uintptr_t)12288;
    struct {
        int got, want;
        const char *what;
    } c[40];
    int n = 0;
#define CASE(call, w) (c[n].got = (call), c[n].want = (w), c[n].what = #call, ++n)
    CASE(sgemm(2, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -1);
    CASE(sgemm(0, 3, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -2);
    CASE(sgemm(0, 0, -1, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -3);
    CASE(sgemm(0, 0, 4, -1, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -4);
    CASE(sgemm(0, 0, 4, 4, -1, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -5);
    CASE(sgemm(0, 0, 4, 4, 4, 1.f, NULL, 4, P, 4, 0.f, P, 4, NULL), -7);
    CASE(sgemm(0, 0, 4, 4, 8, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -8);
    CASE(sgemm(0, 0, 4, 4, 4, 1.f, P, 4, NULL, 4, 0.f, P, 4, NULL), -9);
    CASE(sgemm(0, 0, 4, 8, 4, 1.f, P, 4, P, 4, 0.f, P, 8, NULL), -10);
    CASE(sgemm(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, NULL, 4, NULL), -12);
    CASE(sgemm(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 3, NULL), -13);
    CASE(sgemm_strided_batched(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, -1, 16, 16, 16, NULL),
         -14);
    CASE(sgemm_strided_batched(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 2, -16, 16, 16, NULL),
         -15);
    CASE(sgemm_strided_batched(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 2, 16, -16, 16, NULL),
         -16);
    CASE(sgemm_strided_batched(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 2, 16, 16, -16, NULL),
         -17);
    CASE(sgemm_strided_batched_variant(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 1, 16, 16, 16,
                                       SGEMM_VARIANT_COUNT, NULL),
         -18);
    CASE(sgemm_batched(0, 0, 4, 4, 4, 1.f, NULL, 4, PA, 4, 0.f, PC, 4, 2, NULL), -7);
    CASE(sgemm_batched(0, 0, 4, 4, 4, 1.f, PA, 4, PA, 4, 0.f, PC, 2, 2, NULL), -13);
    CASE(sgemm_colmajor(0, 0, -2, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), -3);
    CASE(sgemm_strided_batched_noalloc(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 1, 16, 16, 16,
                                       -1, NULL),
         -19);
    /* quick returns: nothing to compute, nothing read */
    CASE(sgemm(0, 0, 0, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), 0);
    CASE(sgemm(0, 0, 4, 0, 4, 1.f, P, 4, P, 4, 0.f, P, 4, NULL), 0);
    CASE(sgemm_strided_batched(0, 0, 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 0, 16, 16, 16, NULL), 0);
    CASE(sgemm(0, 0, 4, 4, 0, 1.f, NULL, 1, NULL, 4, 1.f, P, 4, NULL), 0);
    CASE(sgemm(0, 0, 4, 4, 4, 0.f, NULL, 4, NULL, 4, 1.f, P, 4, NULL), 0);
    CASE(sgemm(0, 0, 0, 4, 4, 1.f, NULL, 4, NULL, 4, 0.f, NULL, 4, NULL), 0);
#undef CASE
    for (int i = 0; i < n; ++i)
        CHECK(c[i].got == c[i].want, "%s: %d, want %d", c[i].what, c[i].got, c[i].want);
}

int main(void)
{
    status_strings();
    overrides(300);
    /* the chooser fuzz with a table installed, so every choice looks up */
    {
        int one[7] = {0, 0, 100, 100, 100, 1, SGEMM_VARIANT_S64x64};
        CHECK(sgemm_set_dispatch_overrides(one, 1) == 0, "override table refused");
        dispatch(200000);
        CHECK(sgemm_set_dispatch_overrides(NULL, 0) == 0, "clearing refused");
    }
    windows(2000);
    arguments();
    printf("host checks: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
