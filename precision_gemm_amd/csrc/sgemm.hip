// libsgemm: single-precision GEMM for MI355X (gfx950, CDNA4).
//
//   C = alpha * op(A) @ op(B) + beta * C        (fp32, row-major)
//
// The operation is the SGEMM defined in "From 1% to 94% of cuBLAS, one kernel
// at a time" (the SGEMM paragraph and its kernels' alpha/beta epilogue). The
// structure follows the ideas that page builds up — block tiles staged in
// on-chip memory (kernel 3), register tiles reused across many products
// (kernels 4-5, 10), 128-bit loads (kernel 6), conflict-free shared-memory
// layouts (kernels 7-8), double buffering (its closing list) — and those of
// "Triton Optimization Reference (cuTile -> Triton)": a K loop with no masks
// and the ragged K handled apart (its EVEN_K fast path, section 1; here the
// tile kernels move the partial K-step to the front, so one loop serves every
// K), transposes in the load addressing (section 2), a (tiles, batch) grid
// with grouped tile order (section 3).
//
// How it maps onto CDNA4:
//   * The register tile is a grid of v_mfma_f32_32x32x2_f32 products: full
//     fp32 inputs, fp32 accumulation, 64 lanes per wave. A wave owns a
//     (32*TM) x (32*TN) piece of the workgroup tile.
//   * Each K-step the workgroup copies op(A) (BM x BK) and op(B) (BK x BN)
//     from global memory to LDS with 16-byte buffer loads along whichever
//     dimension is contiguous in memory, so a transposed operand costs
//     nothing extra: only the address map and the LDS layout change.
//       - k-contiguous operand (A with transA=0, B with transB=1): LDS rows
//         of BK floats, one per output row/column, with the 16-byte column
//         XOR-swizzled by row so that 128-bit reads of consecutive rows
//         spread over all 64 LDS banks;
//       - outer-contiguous operand (A with transA=1, B with transB=0): LDS
//         rows of BM (or BN) floats, one per k, read one float per lane.
//   * The k index is permuted inside every group of 8: MFMA step j of a
//     group feeds k = j to lanes 0-31 and k = 4+j to lanes 32-63, so one
//     128-bit LDS read of a k-contiguous row supplies four consecutive MFMA
//     steps. Both operands use the same permutation, so the sum over k is
//     unchanged (only its fp32 rounding order differs).
//   * Masking is free: every load and store goes through a buffer resource
//     whose range ends at the operand's last element; a lane outside M, N or
//     K gets a byte offset >= 2^31, which the hardware turns into a zero load
//     or a dropped store. The resource base advances each K-step, so the
//     per-lane offsets are fixed for the whole loop and stay below 2^31.
//   * LDS is double-buffered with one barrier per K-step; the next step's
//     global loads are in flight while the current step's MFMAs run.
//   * Workgroups are consecutive-ID round-robin over the 8 XCDs; tile IDs are
//     remapped so that each XCD (and its L2) gets a contiguous run of tiles,
//     which are then ordered in groups of GROUP_M tile rows.
//   * Too few tiles to occupy the GPU: the K-split tile runs two wave groups
//     that share each LDS stage and take half its k-groups each (their
//     partial tiles meet in LDS at the end); the split-K entry points cut K
//     across workgroups into a caller workspace and add the slices in a
//     second kernel, always in slice order, so results stay deterministic.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <shared_mutex>
#include <type_traits>
#include <unordered_map>
#include <stdint.h>

#include "sgemm.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kOOB = 0x80000000u;     // any byte offset >= this is out of range
constexpr uint32_t kMaxRange = 0x7fffffffu; // largest buffer range used
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 raw buffer, 32-bit data format
constexpr int kNumXcd = 8;                 // MI355X: 8 XCDs x 32 CUs
// Largest leading dimension for which every in-tile byte offset of the
// buffer-resource kernels, (255*ld + 256)*4 at most, stays below 2^31. Calls
// with a larger one run the 64-bit-addressed tile (the W64x64 variants).
constexpr int kMaxLd = (1 << 21) - 1;

// Batch item b's operands are A + b*sA, B + b*sB, C + b*sC, or, where the
// pointer-array form supplies them, Aarr[b], Barr[b], Carr[b].
struct Params {
    const float *A;
    const float *B;
    float *C;
    const float *const *Aarr;
    const float *const *Barr;
    float *const *Carr;
    int M, N, K;
    int lda, ldb, ldc;
    long long sA, sB, sC;
    float alpha, beta;
    int tiles_m, tiles_n;
    int group_m;
    // Split-K (tile kernels only): with splits > 1, flat batch item b is batch
    // item b / splits and K slice b % splits, covering k in [s*kslice,
    // min((s+1)*kslice, K)); its partial tile goes to C item b.
    int splits, kslice;
    // GEMV kernels only: the first output row of this launch (a launch covers
    // at most 2^31 - 1 work-items, so a very tall matrix takes several).
    int row_base;
    // Persistent kernel only: output tiles per workgroup (one workgroup per
    // compute unit; tiles_m * tiles_n * batch = slot_tiles * workgroups).
    int slot_tiles;
};

__device__ __forceinline__ const float *item_a(const Params &p, int b)
{
    return p.Aarr ? p.Aarr[b] : p.A + b * p.sA;
}
__device__ __forceinline__ const float *item_b(const Params &p, int b)
{
    return p.Barr ? p.Barr[b] : p.B + b * p.sB;
}
__device__ __forceinline__ float *item_c(const Params &p, int b)
{
    return p.Carr ? p.Carr[b] : p.C + b * p.sC;
}

// One output tile the plain way, for a batch item whose A or B pointer does
// not allow the 16-byte loads its kernel was built for (only reachable in the
// pointer-array form, where the host cannot see the item pointers): every
// thread walks whole dot products over k with 4-byte loads.
template <int BM, int BN, int NT, bool A_KC, bool B_KC>
__device__ void plain_tile(const Params &p, const float *Ab, const float *Bb, float *Cb, int K,
                           int m0, int n0)
{
    for (int e = threadIdx.x; e < BM * BN; e += NT) {
        const int i = m0 + e / BN, j = n0 + e % BN;
        if (i >= p.M || j >= p.N)
            continue;
        const long long sa_i = A_KC ? (long long)i * p.lda : i, sa_k = A_KC ? 1 : p.lda;
        const long long sb_j = B_KC ? (long long)j * p.ldb : j, sb_k = B_KC ? 1 : p.ldb;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k)
            acc = __builtin_fmaf(Ab[sa_i + k * sa_k], Bb[sb_j + k * sb_k], acc);
        float *c = Cb + (long long)i * p.ldc + j;
        *c = p.beta == 0.0f ? p.alpha * acc : p.alpha * acc + p.beta * *c;
    }
}

// Buffer range of an operand window that moves `step` bytes per K-step: the
// bytes from the window's start to the end of the operand, capped at
// 2^31 - 1 (the largest range used). While `big` is positive the window is
// still capped; after that `rem` holds the exact bytes left, and stays at 0
// once the window is past the end. Both advance with 32-bit scalar arithmetic
// only. A K loop takes far fewer than 2^31 steps, so `big` saturates at
// INT32_MAX.
struct WindowRange {
    int32_t big, rem, step;

    __host__ __device__ __forceinline__ void init(long long left, int32_t step_bytes)
    {
        step = step_bytes;
        if (left > (long long)kMaxRange) {
            const long long capped = (left - kMaxRange + step_bytes - 1) / step_bytes;
            if (capped >= (long long)INT32_MAX) {
                big = INT32_MAX;
                rem = (int32_t)kMaxRange;
            } else {
                const long long r = left - capped * step_bytes;
                big = (int32_t)capped;
                rem = r < 0 ? 0 : (int32_t)r;
            }
        } else {
            big = 0;
            rem = left < 0 ? 0 : (int32_t)left;
        }
    }
    // Range of the current window, then move to the next one (rem >= 0
    // throughout, so rem - step cannot overflow).
    __host__ __device__ __forceinline__ uint32_t take()
    {
        const bool capped = big > 0;
        const uint32_t range = capped ? kMaxRange : (uint32_t)rem;
        big -= 1;
        rem = capped ? rem : (rem > step ? rem - step : 0);
        return range;
    }
};

// Loads through the global address space (the item pointers arrive as
// generic pointers, which would otherwise become flat loads).
__device__ __forceinline__ f32x4 global_load4(const float *q)
{
    return *(const __attribute__((address_space(1))) f32x4 *)q;
}
__device__ __forceinline__ float global_load1(const float *q)
{
    return *(const __attribute__((address_space(1))) float *)q;
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base, long long elems)
{
    long long bytes = elems * 4;
    uint32_t range = bytes <= 0 ? 0u : (bytes > (long long)kMaxRange ? kMaxRange : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)range,
                                             kRsrcWord3);
}

__device__ __forceinline__ f32x4 load4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// One operand's K-step tile: global -> registers -> LDS, and LDS -> MFMA
// operands. KC: k is the contiguous dimension of the stored operand.
// BO: outer extent of the tile (BM for A, BN for B). VEC: floats per load.
// WIDE: 64-bit element offsets and plain global loads under a per-lane
// predicate instead of 32-bit buffer offsets, for leading dimensions too
// large for the latter (any ld then works; the loop does 64-bit address
// arithmetic, so only calls that need it take this form).
// ---------------------------------------------------------------------------
template <bool KC, int BO, int BK, int NT, int VEC, bool WIDE = false>
struct Operand {
    static constexpr int PAD = 0;                        // outer-contiguous row padding
    static constexpr int ROW = KC ? BK : BO + PAD;       // LDS row length (floats)
    static constexpr int STAGE = KC ? BO * BK : BK * (BO + PAD);
    static constexpr int C4 = KC ? BK / 4 : BO / 4;      // 16-byte chunks per stored tile row
    static constexpr int SLOTS = BO * BK / (4 * NT);     // 16-byte chunks per thread
    static constexpr int EPS = VEC == 4 ? 1 : 4;         // byte offsets kept per slot
    static constexpr int NOFF = SLOTS * EPS;
    // gfx950 serves a 128-bit LDS read from 64 four-byte banks: with k-contiguous
    // rows of BK floats, 64/BK consecutive rows share one sweep of the banks, so
    // the 16-byte chunk index is XORed with (row / (64/BK)) to spread the rows
    // of one read over all banks (measured conflict-free with rocprofv3).
    static constexpr int SWZ_ROWS = BK >= 64 ? 1 : 64 / BK;
    static_assert(BO * BK % (4 * NT) == 0 && SLOTS >= 1, "tile does not split evenly");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert(VEC == 4 || VEC == 1, "VEC");

    const float *X;   // this batch item's operand
    long long ld;
    long long total;  // elements from X to one past the last stored element
    int O, K;         // outer extent and K of the product
    int o0;           // first outer index of this tile
    // Per-lane offsets from the window start: bytes, kOOB for a lane outside
    // the tile's outer range; WIDE: elements, -1 for such a lane.
    std::conditional_t<WIDE, long long, uint32_t> off[NOFF];
    // Window of the next K-step to load: its first element and first k. The
    // first window starts at k = kfirst <= 0, so that a K that is not a
    // multiple of BK leaves its partial step first and every later step full.
    const float *wp;
    int kn;
    WindowRange win;

    __device__ __forceinline__ static int swz(int r) { return (r / SWZ_ROWS) % (BK / 4); }

    // Position of 16-byte chunk (row r, chunk c4) of the K-step tile in LDS.
    __device__ __forceinline__ static int lds_index(int r, int c4)
    {
        return KC ? r * BK + 4 * (c4 ^ swz(r)) : r * ROW + 4 * c4;
    }

    __device__ __forceinline__ void init(int tid, int kfirst)
    {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int f = tid + s * NT, r = f / C4, c4 = f % C4;
            const long long elem = (long long)r * ld + 4 * c4;
#pragma unroll
            for (int e = 0; e < EPS; ++e) {
                // KC: row r is outer index o0+r and the chunk runs along k;
                // otherwise row r is a k index and the chunk runs along outer.
                const bool ok = KC ? (o0 + r < O) : (o0 + 4 * c4 + e < O);
                if constexpr (WIDE)
                    off[s * EPS + e] = ok ? elem + e : -1;
                else
                    off[s * EPS + e] = ok ? (uint32_t)((elem + e) * 4) : kOOB;
            }
        }
        // (kfirst < 0 moves the first window before the tile's k = 0; the
        // lanes there are masked, and the address is formed as an integer.)
        const long long base = (KC ? (long long)o0 * ld : (long long)o0) +
                               (KC ? (long long)kfirst : (long long)kfirst * ld);
        wp = reinterpret_cast<const float *>(reinterpret_cast<uintptr_t>(X) + 4 * base);
        kn = kfirst;
        if constexpr (!WIDE)
            win.init(4 * (total - base), (int32_t)(KC ? 4LL * BK : 4LL * BK * ld));
    }

    // Issue the loads of the next K-step into regs and advance the window.
    // TAIL: also mask k outside [0, K) (needed only for the partial first step).
    template <bool TAIL>
    __device__ __forceinline__ void load_next(int tid, f32x4 (&regs)[SLOTS])
    {
        if constexpr (WIDE) {
            // Every step after the first is full and the first ends inside
            // [0, K), so a step starting at k >= K is wholly past the end
            // (the loads issued ahead of the last steps).
            const bool step_ok = kn < K;
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
                const int f = tid + s * NT, r = f / C4, c4 = f % C4;
                f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int e = 0; e < EPS; ++e) {
                    const long long o = off[s * EPS + e];
                    bool ok = step_ok && o >= 0;
                    if (TAIL)
                        ok = ok && (uint32_t)(KC ? kn + 4 * c4 + (VEC == 4 ? 0 : e) : kn + r) <
                                       (uint32_t)K;
                    if (VEC == 4) {
                        if (ok)
                            v = global_load4(wp + o);
                    } else if (ok) {
                        v[e] = global_load1(wp + o);
                    }
                }
                regs[s] = v;
            }
            wp += KC ? (long long)BK : (long long)BK * ld;
            kn += BK;
            return;
        }
        const uint32_t range = win.take();
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(wp), (short)0, (int)range, kRsrcWord3);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int f = tid + s * NT, r = f / C4, c4 = f % C4;
            if (VEC == 4) {
                uint32_t o = off[s];
                if (TAIL && !((uint32_t)(KC ? kn + 4 * c4 : kn + r) < (uint32_t)K))
                    o |= kOOB;
                regs[s] = load4(rs, o);
            } else {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t o = off[s * 4 + e];
                    if (TAIL && !((uint32_t)(KC ? kn + 4 * c4 + e : kn + r) < (uint32_t)K))
                        o |= kOOB;
                    v[e] = load1(rs, o);
                }
                regs[s] = v;
            }
        }
        wp += KC ? (long long)BK : (long long)BK * ld;
        kn += BK;
    }

    __device__ __forceinline__ static void store(float *lds, int tid, const f32x4 (&regs)[SLOTS])
    {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int f = tid + s * NT, r = f / C4, c4 = f % C4;
            *reinterpret_cast<f32x4 *>(lds + lds_index(r, c4)) = regs[s];
        }
    }

    // MFMA operands of k-group q (8 k values) for the 32-row slab at outer
    // offset w (inside the tile): v[j] feeds MFMA step j of the group. Kept as
    // four scalars so every LDS read result feeds its MFMA directly.
    __device__ __forceinline__ static void frag(const float *lds, int w, int q, int lane,
                                                float (&v)[4])
    {
        const int o = w + (lane & 31), g = lane >> 5;
        if (KC) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(lds + lds_index(o, 2 * q + g));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = x[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = lds[(8 * q + 4 * g + j) * ROW + o];
        }
    }
};

// Logical tile index -> (batch item, tile row, tile column): items one after
// another, each in grouped order.
__device__ __forceinline__ void decode_tile(const Params &p, int logical, int &b, int &tm, int &tn)
{
    const int per_batch = p.tiles_m * p.tiles_n;
    b = logical / per_batch;
    const int t = logical % per_batch;
    // Grouped order: GROUP_M tile rows are walked column by column.
    const int in_group = p.group_m * p.tiles_n;
    const int first_m = (t / in_group) * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    tm = first_m + (t % in_group) % gsize;
    tn = (t % in_group) / gsize;
}

// Flat workgroup id -> (batch item, tile row, tile column).
__device__ __forceinline__ void tile_of(const Params &p, int &b, int &tm, int &tn)
{
    const int num = gridDim.x * gridDim.y;
    const int pid = blockIdx.y * gridDim.x + blockIdx.x;
    // Workgroup pid runs on XCD pid % 8; give each XCD a contiguous range.
    const int xcd = pid % kNumXcd, local = pid / kNumXcd;
    const int q = num / kNumXcd, r = num % kNumXcd;
    const int logical = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    decode_tile(p, logical, b, tm, tn);
}

// Epilogue of a tile kernel: C = alpha * res + beta * C for this wave's
// outputs, lanes outside M x N dropped (C is not read when beta == 0).
// res[i][j][vv] is accumulator register v0 + vv of the wave's MFMA tile (i, j):
// register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the
// 32 x 32 product at (wm0 + 32 i, wn0 + 32 j) inside the workgroup tile.
template <int TM, int TN, int VN, bool WIDE = false>
__device__ __forceinline__ void store_tile(const Params &p, float *Cb, int m0, int n0, int wm0,
                                           int wn0, int v0, int lane,
                                           const float (&res)[TM][TN][VN])
{
    if constexpr (WIDE) {
        // 64-bit addresses; lanes outside M x N store nothing.
        const int g = lane >> 5;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int vv = 0; vv < VN; ++vv) {
                    const int v = v0 + vv;
                    const int row = m0 + wm0 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
                    const int col = n0 + wn0 + 32 * j + (lane & 31);
                    if (row < p.M && col < p.N) {
                        float *c = Cb + (long long)row * p.ldc + col;
                        *c = p.beta == 0.0f ? p.alpha * res[i][j][vv]
                                            : __builtin_fmaf(p.alpha, res[i][j][vv], p.beta * *c);
                    }
                }
        return;
    }
    const long long cbase = (long long)m0 * p.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(Cb + cbase, (long long)(p.M - 1) * p.ldc + p.N - cbase);
    const int g = lane >> 5;
    auto epilogue = [&](auto with_beta) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = wn0 + 32 * j + (lane & 31);
                const bool col_ok = n0 + col < p.N;
                uint32_t off[VN];
                float c[VN];
#pragma unroll
                for (int vv = 0; vv < VN; ++vv) {
                    const int v = v0 + vv;
                    const int row = wm0 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
                    off[vv] = (col_ok && m0 + row < p.M)
                                  ? (uint32_t)(((long long)row * p.ldc + col) * 4)
                                  : kOOB;
                    if (with_beta)
                        c[vv] = load1(rc, off[vv]);
                }
                // alpha * acc, or fma(alpha, acc, beta * c): one rounding
                // order for every tile kernel, whatever the compiler contracts.
#pragma unroll
                for (int vv = 0; vv < VN; ++vv) {
                    const float out = with_beta
                                          ? __builtin_fmaf(p.alpha, res[i][j][vv], p.beta * c[vv])
                                          : p.alpha * res[i][j][vv];
                    store1(rc, off[vv], out);
                }
            }
        }
    };
    if (p.beta != 0.0f)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// WAVES_K = 2 splits every K-step between two groups of WAVES_M x WAVES_N
// waves: group g multiplies the k-groups [g*NQ/2, (g+1)*NQ/2) of each stage
// into its own accumulators, which gives every SIMD two waves on a tile that
// would otherwise leave one. The two partial tiles are added through LDS at
// the end in a fixed order (group 0's plus group 1's), so results do not
// depend on timing.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int WAVES_K, int MIN_WAVES_PER_EU,
          bool A_KC, bool B_KC, int VEC, bool WIDE>
__global__ void
__attribute__((amdgpu_flat_work_group_size(64 * WAVES_M * WAVES_N * WAVES_K,
                                           64 * WAVES_M * WAVES_N * WAVES_K),
               amdgpu_waves_per_eu(MIN_WAVES_PER_EU)))
sgemm_mfma_kernel(Params p)
{
    constexpr int WAVES_MN = WAVES_M * WAVES_N;
    constexpr int NT = 64 * WAVES_MN * WAVES_K;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(WAVES_K == 1 || WAVES_K == 2, "WAVES_K");
    using OpA = Operand<A_KC, BM, BK, NT, VEC, WIDE>;
    using OpB = Operand<B_KC, BN, BK, NT, VEC, WIDE>;

    // Two stages, each holding the A tile followed by the B tile.
    constexpr int STAGE = OpA::STAGE + OpB::STAGE;
    __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

    int b, tile_m, tile_n;
    tile_of(p, b, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wmn = wave % WAVES_MN, kgrp = wave / WAVES_MN;
    const int wm0 = (wmn % WAVES_M) * WM, wn0 = (wmn / WAVES_M) * WN;

    // This workgroup's K range: the whole K, or its slice under split-K (the
    // slice's operands start k0 into A and B; kslice is a multiple of BK).
    int item = b, k0 = 0, Kt = p.K;
    if (p.splits > 1) {
        item = b / p.splits;
        k0 = (b - item * p.splits) * p.kslice;
        Kt = min(p.kslice, p.K - k0);
    }
    const float *Ab = item_a(p, item) + (A_KC ? (long long)k0 : (long long)k0 * p.lda);
    const float *Bb = item_b(p, item) + (B_KC ? (long long)k0 : (long long)k0 * p.ldb);
    float *Cb = item_c(p, b);
    if (VEC == 4 && (((uintptr_t)Ab | (uintptr_t)Bb) & 15u)) {
        plain_tile<BM, BN, NT, A_KC, B_KC>(p, Ab, Bb, Cb, Kt, m0, n0);
        return;
    }

    OpA opa;
    opa.X = Ab;
    opa.ld = p.lda;
    opa.total = A_KC ? (long long)(p.M - 1) * p.lda + Kt : (long long)(Kt - 1) * p.lda + p.M;
    opa.O = p.M;
    opa.K = Kt;
    opa.o0 = m0;
    // A K that is not a multiple of BK puts its partial step first.
    const int kfirst = Kt % BK == 0 ? 0 : Kt % BK - BK;
    opa.init(tid, kfirst);
    OpB opb;
    opb.X = Bb;
    opb.ld = p.ldb;
    opb.total = B_KC ? (long long)(p.N - 1) * p.ldb + Kt : (long long)(Kt - 1) * p.ldb + p.N;
    opb.O = p.N;
    opb.K = Kt;
    opb.o0 = n0;
    opb.init(tid, kfirst);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    // LATE_STORE: two register buffers for the staged
    // loads, by step parity. Step s issues the loads of step s + 2 first and
    // writes step s + 1's data (loaded one step earlier) to LDS halfway
    // through its MFMAs, so a load has about one and a half steps to arrive
    // instead of one: operands streamed from HBM rather than the Infinity
    // Cache then arrive in time (4092^3 with operands not cached: 1.14 ms
    // with the writes at the start of the step, 0.93 ms with them halfway;
    // at the end of the step the warm case lost 1 %, as the writes then
    // delay the barrier).
    constexpr bool LATE_STORE = !WIDE;
    constexpr int NBUF = LATE_STORE ? 2 : 1;
    f32x4 ra[NBUF][OpA::SLOTS], rb[NBUF][OpB::SLOTS];
    const int nsteps = (Kt + BK - 1) / BK;

    // Every K-step after the first is full, so only the prologue's first load
    // carries a k mask (a no-op when K is a multiple of BK): the K loop is the
    // same code for every K. (With a partial last step instead, the masked
    // copy of the kernel compiled to a schedule 24 % slower for two
    // k-contiguous operands.)
    using Masked = std::true_type;
    using Full = std::false_type;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, NBUF - 1>;
    auto load = [&](auto tail, auto buf) {
        opa.template load_next<decltype(tail)::value>(tid, ra[decltype(buf)::value]);
        opb.template load_next<decltype(tail)::value>(tid, rb[decltype(buf)::value]);
    };

    constexpr int NQ = BK / 8 / WAVES_K; // groups of 8 k per K-step, per wave
    constexpr int LATE = TM * TN;        // MFMAs of the last group issued after the barrier
    static_assert(NQ >= 2, "the fragment pipeline needs at least two k-groups per step");
    const int q0 = kgrp * NQ;            // this wave's first k-group of a stage

    auto read_group = [&](const float *stage, int q, float (&fa)[TM][4], float (&fb)[TN][4]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            OpA::frag(stage, wm0 + 32 * i, q0 + q, lane, fa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            OpB::frag(stage + OpA::STAGE, wn0 + 32 * j, q0 + q, lane, fb[j]);
    };
    // MFMA steps [first, last) of one k-group, step-major so that consecutive
    // MFMAs update different accumulators.
    auto mfma_group = [&](const float (&fa)[TM][4], const float (&fb)[TN][4], int first, int last) {
#pragma unroll
        for (int t = 0; t < 4 * TM * TN; ++t) {
            if (t < first || t >= last)
                continue;
            const int kk = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk], fb[j][kk], acc[i][j],
                                                              0, 0, 0);
        }
    };

    load(Masked{}, B0{});
    OpA::store(lds, tid, ra[0]);
    OpB::store(lds + OpA::STAGE, tid, rb[0]);
    load(Full{}, B1{});
    __syncthreads();

    // Software pipeline over K-steps. Group 0 of a stage is read right after
    // the barrier that publishes it, while the previous step's last MFMAs are
    // still being issued; the other groups are read while group 0's MFMAs run.
    // The next stage's LDS writes and the global loads two steps ahead go
    // between MFMA groups. One barrier per step. The step is written for a
    // fixed stage parity, so every LDS address is a loop-invariant register
    // plus an immediate offset and the loop body does no address arithmetic.
    float fa[NQ][TM][4], fb[NQ][TN][4];
    read_group(lds, 0, fa[0], fb[0]);
    auto k_step = [&](auto parity, auto tail) {
        constexpr int PAR = decltype(parity)::value;
        const float *cur = lds + PAR * STAGE;
        float *nxt = lds + (1 - PAR) * STAGE;
#pragma unroll
        for (int q = 1; q < NQ; ++q)
            read_group(cur, q, fa[q], fb[q]);
        mfma_group(fa[0], fb[0], 0, 4 * TM * TN);
        // The stage written here is idle this step. On the last two steps the
        // writes and loads are of no use but harmless (their windows lie past
        // the last K-step; a lane reads either memory inside the operand's
        // buffer range or, beyond it, zeros).
        constexpr int NW = OpA::SLOTS + OpB::SLOTS;      // LDS writes
        constexpr int NL = NW * OpA::EPS;                // global loads
        constexpr int NM = 4 * TM * TN * NQ - LATE;      // MFMAs before the barrier
        if constexpr (LATE_STORE) {
            // Loads of step s + 2 into the buffer step s's data left, then the
            // MFMAs, with step s + 1's data written to LDS halfway through them.
            load(tail, std::integral_constant<int, PAR>{});
#pragma unroll
            for (int q = 1; q < NQ - 1; ++q)
                mfma_group(fa[q], fb[q], 0, 4 * TM * TN);
            mfma_group(fa[NQ - 1], fb[NQ - 1], 0, 4 * TM * TN - LATE);
            OpA::store(nxt, tid, ra[1 - PAR]);
            OpB::store(nxt + OpA::STAGE, tid, rb[1 - PAR]);
            // Order: this stage's remaining fragment reads, MFMAs alternating
            // with the global loads, MFMAs, MFMAs alternating with the writes,
            // the rest of the MFMAs.
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN) * (NQ - 1), 0);
#pragma unroll
            for (int w = 0; w < NL; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // global load
            }
            constexpr int MID = (NM - NL - NW) / 2 > 0 ? (NM - NL - NW) / 2 : 0;
            if constexpr (MID > 0)
                __builtin_amdgcn_sched_group_barrier(0x008, MID, 0);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // LDS write
            }
        } else {
            OpA::store(nxt, tid, ra[0]);
            OpB::store(nxt + OpA::STAGE, tid, rb[0]);
            load(tail, B0{});
#pragma unroll
            for (int q = 1; q < NQ - 1; ++q)
                mfma_group(fa[q], fb[q], 0, 4 * TM * TN);
            mfma_group(fa[NQ - 1], fb[NQ - 1], 0, 4 * TM * TN - LATE);
            // Order: this stage's remaining fragment reads, then MFMAs
            // alternating with the next stage's LDS writes and the global loads.
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN) * (NQ - 1), 0);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // LDS write
            }
#pragma unroll
            for (int w = 0; w < NL; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // global load
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // (On the last step this reads the idle stage; the values are unused.)
        read_group(nxt, 0, fa[0], fb[0]);
        mfma_group(fa[NQ - 1], fb[NQ - 1], 4 * TM * TN - LATE, 4 * TM * TN);
        // Issue the reads first so their latency runs under the late MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN), 0); // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, LATE, 0);          // MFMAs
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // Step s loads step s + 2 (the loads of the last two steps read nothing
    // that is used), two steps per trip.
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        k_step(P0{}, Full{});
        k_step(P1{}, Full{});
    }
    // An odd last step (the pairs above end on an even step: parity 0).
    if (s < nsteps)
        k_step(P0{}, Full{});

    // Accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
    // column l%32 of its 32 x 32 product. With WAVES_K = 2, wave group h
    // finishes registers [8h, 8h+8) of every tile: it receives the other
    // group's partial sums of those through LDS and sends its own of the rest.
    constexpr int VN = 16 / WAVES_K;     // accumulator registers finished per wave
    const int v0 = kgrp * VN;
    float res[TM][TN][VN];
    if constexpr (WAVES_K == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < VN; ++v)
                    res[i][j][v] = acc[i][j][v];
    } else {
        static_assert(BM * BN <= 2 * STAGE, "the exchange must fit in the stages' LDS");
        // Slot of (receiving group r, this wave's tile position, register v - 8r, lane).
        auto xidx = [&](int r, int i, int j, int vv) {
            return ((((r * WAVES_MN + wmn) * TM + i) * TN + j) * VN + vv) * 64 + lane;
        };
        __syncthreads(); // every wave is past its last read of the stages
        const int other = 1 - kgrp;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int vv = 0; vv < VN; ++vv)
                    lds[xidx(other, i, j, vv)] = kgrp == 0 ? acc[i][j][VN + vv] : acc[i][j][vv];
        __syncthreads();
        // Group 0's partial plus group 1's, in that order for either group
        // (the sum of two floats does not depend on the operand order).
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int vv = 0; vv < VN; ++vv) {
                    const float mine = kgrp == 0 ? acc[i][j][vv] : acc[i][j][VN + vv];
                    res[i][j][vv] = mine + lds[xidx(kgrp, i, j, vv)];
                }
    }

    store_tile<TM, TN, VN, WIDE>(p, Cb, m0, n0, wm0, wn0, v0, lane, res);
}

// ---------------------------------------------------------------------------
// Persistent tile kernel: one workgroup per compute unit, looping over that
// unit's output tiles, the pattern "Triton Optimization Reference (cuTile ->
// Triton)" describes for persistent kernels (a grid sized to the machine,
// each program walking tiles in grouped order). The workgroup is twelve
// waves, three groups of 2 x 2 waves that each own a BM x BN accumulator, so
// every SIMD runs three waves as with three workgroups per CU. A unit with n
// tiles, n = 3q + 1, gives each group q whole tiles and then a third of the K
// range of the last one (the stream-K split of a ragged last round, kept
// inside the CU): the three partial tiles are added in LDS in a fixed order,
// (group 0 + group 1) + group 2, so results do not depend on timing. Every
// group runs the same number of K-steps in every tile, so the workgroup-wide
// barriers of the K loop line up by construction: no group ever waits at a
// barrier the others do not reach. A third of K is a piece of L_g k (L_1 =
// L_2 = K/3 rounded up to a multiple of 4, L_0 the rest), all run as the same
// number of 16-deep steps P: a piece's first window starts L_g - 16P before
// its end (up to 31 k before its start), and the first two loads of every
// tile mask k outside [0, L_g). Tiles on one XCD (workgroup pid runs on XCD
// pid % 8) are a contiguous range of the grouped order, and the groups of the
// XCD's workgroups take consecutive tiles of it at the same time.
// ---------------------------------------------------------------------------
template <int BM, int BN, bool A_KC, bool B_KC>
__global__ void __attribute__((amdgpu_flat_work_group_size(768, 768), amdgpu_waves_per_eu(3)))
sgemm_persistent_kernel(Params p)
{
    constexpr int BK = 16, NT = 256, GROUPS = 3;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int NQ = BK / 8, LATE = TM * TN;
    using OpA = Operand<A_KC, BM, BK, NT, 4>;
    using OpB = Operand<B_KC, BN, BK, NT, 4>;
    constexpr int STAGE = OpA::STAGE + OpB::STAGE;
    constexpr int PART = 4 * TM * TN * 16 * 64; // one group's accumulators
    constexpr int LDS = GROUPS * 2 * STAGE > 2 * PART ? GROUPS * 2 * STAGE : 2 * PART;
    __shared__ __attribute__((aligned(16))) float lds[LDS];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / 4, wg = wave % 4;
    const int wm0 = (wg % 2) * WM, wn0 = (wg / 2) * WN;
    float *stages = lds + grp * 2 * STAGE;

    // This workgroup's tiles: XCD x owns the logical tiles
    // [x * per_xcd, (x + 1) * per_xcd); its workgroup l takes, in round u,
    // local tile (3u + g) * slots_x + l for group g, and the split tile
    // 3q * slots_x + l.
    const int pid = blockIdx.x, slots = gridDim.x;
    const int slots_x = slots / kNumXcd, xcd = pid % kNumXcd, l = pid / kNumXcd;
    const int n = p.slot_tiles, q = n / 3;
    const int first = xcd * slots_x * n;

    const int K = p.K;
    const int steps_whole = (K + BK - 1) / BK;
    const int piece = 4 * ((K + 11) / 12);           // L_1 = L_2
    const int my_k0 = grp == 0 ? 0 : K - (GROUPS - grp) * piece;
    const int my_len = grp == 0 ? K - 2 * piece : piece;
    const int steps_piece = (piece + BK - 1) / BK;   // P (L_0 <= L_1)

    f32x16 acc[TM][TN];
    // One tile: the product of op(A)[m0.., k0..k0+len) and op(B)[k0..k0+len,
    // n0..) over `steps` K-steps into acc (cleared first).
    auto run_unit = [&](int lane, int b, int m0, int n0, int k0, int len, int steps) {
        const int tid = wg * 64 + lane;
        const float *Ab = item_a(p, b) + (A_KC ? (long long)k0 : (long long)k0 * p.lda);
        const float *Bb = item_b(p, b) + (B_KC ? (long long)k0 : (long long)k0 * p.ldb);
        OpA opa;
        opa.X = Ab;
        opa.ld = p.lda;
        opa.total = A_KC ? (long long)(p.M - 1) * p.lda + len : (long long)(len - 1) * p.lda + p.M;
        opa.O = p.M;
        opa.K = len;
        opa.o0 = m0;
        const int kfirst = len - BK * steps;
        opa.init(tid, kfirst);
        OpB opb;
        opb.X = Bb;
        opb.ld = p.ldb;
        opb.total = B_KC ? (long long)(p.N - 1) * p.ldb + len : (long long)(len - 1) * p.ldb + p.N;
        opb.O = p.N;
        opb.K = len;
        opb.o0 = n0;
        opb.init(tid, kfirst);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = f32x16{};
        f32x4 ra[OpA::SLOTS], rb[OpB::SLOTS];
        using Masked = std::true_type;
        using Full = std::false_type;
        auto load = [&](auto tail) {
            opa.template load_next<decltype(tail)::value>(tid, ra);
            opb.template load_next<decltype(tail)::value>(tid, rb);
        };
        auto read_group = [&](const float *stage, int qq, float (&fa)[TM][4], float (&fb)[TN][4]) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                OpA::frag(stage, wm0 + 32 * i, qq, lane, fa[i]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                OpB::frag(stage + OpA::STAGE, wn0 + 32 * j, qq, lane, fb[j]);
        };
        auto mfma_group = [&](const float (&fa)[TM][4], const float (&fb)[TN][4], int lo, int hi) {
#pragma unroll
            for (int t = 0; t < 4 * TM * TN; ++t) {
                if (t < lo || t >= hi)
                    continue;
                const int kk = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk], fb[j][kk], acc[i][j],
                                                                  0, 0, 0);
            }
        };
        // Both prologue loads mask k outside [0, len): a piece's first window
        // may start up to 31 k before it.
        load(Masked{});
        OpA::store(stages, tid, ra);
        OpB::store(stages + OpA::STAGE, tid, rb);
        load(Masked{});
        __syncthreads();
        float fa[NQ][TM][4], fb[NQ][TN][4];
        read_group(stages, 0, fa[0], fb[0]);
        auto k_step = [&](auto parity) {
            constexpr int PAR = decltype(parity)::value;
            const float *cur = stages + PAR * STAGE;
            float *nxt = stages + (1 - PAR) * STAGE;
#pragma unroll
            for (int qq = 1; qq < NQ; ++qq)
                read_group(cur, qq, fa[qq], fb[qq]);
            mfma_group(fa[0], fb[0], 0, 4 * TM * TN);
            OpA::store(nxt, tid, ra);
            OpB::store(nxt + OpA::STAGE, tid, rb);
            load(Full{});
#pragma unroll
            for (int qq = 1; qq < NQ - 1; ++qq)
                mfma_group(fa[qq], fb[qq], 0, 4 * TM * TN);
            mfma_group(fa[NQ - 1], fb[NQ - 1], 0, 4 * TM * TN - LATE);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN) * (NQ - 1), 0);
#pragma unroll
            for (int w = 0; w < OpA::SLOTS + OpB::SLOTS; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // LDS write
            }
#pragma unroll
            for (int w = 0; w < OpA::SLOTS + OpB::SLOTS; ++w) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // global load
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            read_group(nxt, 0, fa[0], fb[0]);
            mfma_group(fa[NQ - 1], fb[NQ - 1], 4 * TM * TN - LATE, 4 * TM * TN);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN), 0);
            __builtin_amdgcn_sched_group_barrier(0x008, LATE, 0);
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        int s = 0;
        for (; s + 1 < steps; s += 2) {
            k_step(P0{});
            k_step(P1{});
        }
        if (s < steps)
            k_step(P0{});
    };

    // Tiles: q whole ones, then (n % 3 == 1) this group's third of the split
    // tile. The split tile is the same for the whole workgroup, so the
    // barriers of its exchange are reached by every wave.
    const int units = q + (n - 3 * q == 1 ? 1 : 0);
    for (int u = 0; u < units; ++u) {
        // The lane index, opaque to the compiler in every tile: the per-lane
        // load, LDS and store offsets are then recomputed per tile instead of
        // hoisted out of this loop and held (spilled) across the K loop.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const bool split = u == q;
        int b, tm, tn;
        decode_tile(p, first + (split ? 3 * q : 3 * u + grp) * slots_x + l, b, tm, tn);
        run_unit(lane, b, tm * BM, tn * BN, split ? my_k0 : 0, split ? my_len : K,
                 split ? steps_piece : steps_whole);
        if (split) {
            // Groups 0 and 1 hand their partial tiles to group 2, which adds
            // (group 0 + group 1) + its own and stores the tile.
            auto xidx = [&](int g, int i, int j, int v) {
                return ((((g * 4 + wg) * TM + i) * TN + j) * 16 + v) * 64 + lane;
            };
            __syncthreads(); // every wave is past its last read of the stages
            if (grp < 2) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            lds[xidx(grp, i, j, v)] = acc[i][j][v];
            }
            __syncthreads();
            if (grp == 2) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[i][j][v] = (lds[xidx(0, i, j, v)] + lds[xidx(1, i, j, v)]) +
                                           acc[i][j][v];
            }
        }
        if (!split || grp == 2) {
            float res[TM][TN][16];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        res[i][j][v] = acc[i][j][v];
            store_tile<TM, TN, 16>(p, item_c(p, b), tm * BM, tn * BN, wm0, wn0, 0, lane, res);
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel for grids of few tiles over a deep K (never launched with
// split-K): a BM x 64 tile per workgroup whose WAVES waves each own every
// WAVES-th K-step (wave w takes steps w, w+WAVES, ...) and accumulate the
// whole tile over their steps. Two configurations: 64 x 64 with four waves
// and 4-deep rings, for a skinny dimension whose long operand streams from
// HBM, and 32 x 64 with eight waves (two per SIMD) and 3-deep rings, for
// grids of at most one such tile per CU, where a call lasts as long as one
// workgroup's tile. Every
// wave fills its own ring of STAGES LDS buffers with direct-to-LDS 16-byte
// buffer loads (buffer_load_dwordx4 ... lds: lane i of an instruction writes
// the i-th 16 bytes of a 1 KiB block, an out-of-range lane writes zeros) and
// reads back only what it loaded itself, so the K loop needs no barrier: a
// wave waits on its own vmcnt only. Loads run STAGES-1 steps ahead, which
// keeps enough bytes in flight per CU to stream the long operand at HBM rate.
// At the end the partial tiles are summed through LDS in a fixed order
// (deterministic) and the alpha/beta epilogue is applied.
// ---------------------------------------------------------------------------
// NW waves share each K-step tile: wave w loads blocks w, w + NW, ... (NW = 1:
// a wave loads its whole tile).
template <bool KC, int BO, int BK, int NW = 1>
struct DmaOperand {
    static constexpr int FLOATS = BO * BK;         // one K-step tile
    static constexpr int NINST = FLOATS * 4 / 1024; // 1 KiB blocks, one load instruction each
    static constexpr int NBW = NINST / NW;          // blocks loaded by each wave
    static constexpr int C4 = KC ? BK / 4 : BO / 4; // 16-byte chunks per stored row of the tile
    static constexpr int SWZ_ROWS = BK >= 64 ? 1 : 64 / BK;
    static_assert(FLOATS * 4 % 1024 == 0, "tile must be whole 1 KiB blocks");
    static_assert(NINST % NW == 0, "blocks must split evenly over the waves");

    const float *X;
    long long ld, total;
    int O, K, o0;
    int wv;               // this wave's index among the NW sharing the tile
    uint32_t off[NBW];    // this lane's chunk in each of its blocks, relative to the step's window
    // Window of this wave's next K-step (the waves of a workgroup take every
    // WAVES-th step): first element and first k, and its buffer range.
    const float *wp;
    int kn, kstep;
    WindowRange win;
    long long step_elems;

    __device__ __forceinline__ static int swz(int r) { return (r / SWZ_ROWS) % (BK / 4); }

    // Block b, lane: LDS chunk position f = 64 b + lane. KC: row f / C4 holds
    // logical chunk (f % C4) ^ swz(row); otherwise row f / C4 (a k) holds
    // chunk f % C4 (four outer indices).
    __device__ __forceinline__ void chunk(int b, int lane, int &r, int &c) const
    {
        const int f = 64 * b + lane;
        r = f / C4;
        c = KC ? (f % C4) ^ swz(r) : f % C4;
    }

    // k0: first k of this wave's first step; kstride: k between its steps.
    __device__ __forceinline__ void init(int lane, int k0, int kstride, int wave_in_tile = 0)
    {
        wv = wave_in_tile;
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            int r, c;
            chunk(wv + NW * i, lane, r, c);
            const bool ok = KC ? (o0 + r < O) : (o0 + 4 * c < O);
            off[i] = ok ? (uint32_t)(((long long)r * ld + 4 * c) * 4) : kOOB;
        }
        // (k0 < 0: the window starts before the tile's k = 0; those lanes are
        // masked, and the address is formed as an integer.)
        const long long base = KC ? (long long)o0 * ld + k0 : (long long)k0 * ld + o0;
        wp = reinterpret_cast<const float *>(reinterpret_cast<uintptr_t>(X) + 4 * base);
        kn = k0;
        kstep = kstride;
        step_elems = KC ? (long long)kstride : (long long)kstride * ld;
        win.init(4 * (total - base), (int32_t)(4 * step_elems));
    }

    // Load this wave's next K-step into `tile` and advance the window.
    // TAIL: also mask k outside [0, K) (needed only for a first window that
    // starts before k = 0).
    template <bool TAIL>
    __device__ __forceinline__ void issue(float *tile, int lane)
    {
        const uint32_t range = win.take();
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(wp), (short)0, (int)range, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wv + NW * i;
            uint32_t o = off[i];
            if (TAIL) {
                int r, c;
                chunk(b, lane, r, c);
                if (!((uint32_t)(KC ? kn + 4 * c : kn + r) < (uint32_t)K))
                    o |= kOOB;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)(tile + 256 * b), 16, o, 0, 0, 0);
        }
        wp += step_elems;
        kn += kstep;
    }

    // Same operand layout contract as Operand::frag (k permuted within groups of 8).
    __device__ __forceinline__ static void frag(const float *tile, int w, int q, int lane,
                                                float (&v)[4])
    {
        const int o = w + (lane & 31), g = lane >> 5;
        if (KC) {
            const int c = 2 * q + g;
            const f32x4 x =
                *reinterpret_cast<const f32x4 *>(tile + o * BK + 4 * (c ^ swz(o)));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = x[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = tile[(8 * q + 4 * g + j) * BO + o];
        }
    }
};

// Wait until at most min(n, MAXN) groups of NI vector-memory operations are in
// flight (n < 0: none). n is wave-uniform; each case has its own immediate.
template <int NI, int MAXN>
__device__ __forceinline__ void wait_vm_groups(int n)
{
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(MAXN * NI));
            return;
        }
        wait_vm_groups<NI, MAXN - 1>(n);
    } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
}

template <int WAVES, int STAGES, int BM, int BN, int MINW, bool A_KC, bool B_KC>
__global__ void
__attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES), amdgpu_waves_per_eu(MINW)))
sgemm_stream_kernel(Params p)
{
    constexpr int BK = 16, TM = BM / 32, TN = BN / 32, NQ = BK / 8;
    // Epilogue: a wave covers 64 / BN rows per pass (one column per lane).
    constexpr int RPW = 64 / BN;
    constexpr int RPT = BM / (WAVES * RPW); // epilogue rows per thread
    using OpA = DmaOperand<A_KC, BM, BK>;
    using OpB = DmaOperand<B_KC, BN, BK>;
    constexpr int STAGE = OpA::FLOATS + OpB::FLOATS;      // floats per ring slot
    constexpr int NI = OpA::NINST + OpB::NINST;           // load instructions per step
    constexpr int PITCH = BN + 4;                         // partial-tile row pitch
    constexpr int RING = WAVES * STAGES * STAGE;
    constexpr int PART = WAVES * BM * PITCH;
    static_assert((STAGES - 2) * NI <= 63 && RPT <= 63, "vmcnt holds at most 63");
    static_assert((BN == 64 || BN == 32) && BM % (WAVES * RPW) == 0, "epilogue split");
    __shared__ __attribute__((aligned(16))) float lds[RING > PART ? RING : PART];

    int b, tile_m, tile_n;
    tile_of(p, b, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    // The wave index is uniform across the wave; saying so keeps the LDS
    // destination of the direct loads (M0) a scalar.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const float *Ab = item_a(p, b), *Bb = item_b(p, b);
    float *Cb = item_c(p, b);
    if (((uintptr_t)Ab | (uintptr_t)Bb) & 15u) {
        plain_tile<BM, BN, 64 * WAVES, A_KC, B_KC>(p, Ab, Bb, Cb, p.K, m0, n0);
        return;
    }

    OpA opa;
    opa.X = Ab;
    opa.ld = p.lda;
    opa.total = A_KC ? (long long)(p.M - 1) * p.lda + p.K : (long long)(p.K - 1) * p.lda + p.M;
    opa.O = p.M;
    opa.K = p.K;
    opa.o0 = m0;
    // A K that is not a multiple of BK puts its partial step first (wave 0's
    // first step): only the first load of each wave carries a k mask.
    const int kfirst = p.K % BK == 0 ? 0 : p.K % BK - BK;
    opa.init(lane, kfirst + wave * BK, WAVES * BK);
    OpB opb;
    opb.X = Bb;
    opb.ld = p.ldb;
    opb.total = B_KC ? (long long)(p.N - 1) * p.ldb + p.K : (long long)(p.K - 1) * p.ldb + p.N;
    opb.O = p.N;
    opb.K = p.K;
    opb.o0 = n0;
    opb.init(lane, kfirst + wave * BK, WAVES * BK);

    float *ring = lds + wave * STAGES * STAGE;
    // My j-th step is K-step wave + WAVES j; its loads go to ring slot j % STAGES.
    auto issue = [&](int j, auto masked) {
        float *slot = ring + (j % STAGES) * STAGE;
        opa.template issue<decltype(masked)::value>(slot, lane);
        opb.template issue<decltype(masked)::value>(slot + OpA::FLOATS, lane);
    };
    float fa[2][NQ][TM][4], fb[2][NQ][TN][4];
    auto read = [&](int j, float (&xa)[NQ][TM][4], float (&xb)[NQ][TN][4]) {
        const float *slot = ring + (j % STAGES) * STAGE;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                OpA::frag(slot, 32 * i, q, lane, xa[q][i]);
#pragma unroll
            for (int t = 0; t < TN; ++t)
                OpB::frag(slot + OpA::FLOATS, 32 * t, q, lane, xb[q][t]);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
            acc[i][t] = f32x16{};

    // Loads run STAGES - 1 steps ahead of the MFMAs and stop at the wave's
    // last step; waiting for step s leaves the loads of the steps issued after
    // it in flight (vector-memory operations complete in issue order).
    const int nsteps = (p.K + BK - 1) / BK;
    const int mine = wave < nsteps ? (nsteps - wave + WAVES - 1) / WAVES : 0;
    if (mine > 0)
        issue(0, std::true_type{});
#pragma unroll
    for (int j = 1; j < STAGES - 1; ++j)
        if (j < mine)
            issue(j, std::false_type{});
    wait_vm_groups<NI, STAGES - 2>(mine - 1);
    read(0, fa[0], fb[0]);
    // Step i: issue step i + STAGES - 1 (if it exists), wait for step i + 1,
    // read it into the other register buffer, multiply step i. H is i's
    // parity, so the register double buffer has static indices.
    auto step = [&](auto h, auto steady, int i) {
        constexpr int H = decltype(h)::value;
        if (decltype(steady)::value) {
            issue(i + STAGES - 1, std::false_type{});
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((STAGES - 2) * NI));
        } else if (i + STAGES - 1 < mine) {
            issue(i + STAGES - 1, std::false_type{});
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((STAGES - 2) * NI));
        } else {
            wait_vm_groups<NI, STAGES - 2>(mine - 2 - i); // steps issued after i + 1
        }
        // (After the last step this reads a slot whose values are unused.)
        read(i + 1, fa[H ^ 1], fb[H ^ 1]);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ii = 0; ii < TM; ++ii)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[ii][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            fa[H][q][ii][kk], fb[H][q][t][kk], acc[ii][t], 0, 0, 0);
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    // Steady state: every step issues a load and waits a fixed count; one
    // basic block per trip, so the loads interleave with the MFMAs.
    const int steady_end = mine - (STAGES - 1);
    int i = 0;
    for (; i + 1 < steady_end; i += 2) {
        step(H0{}, std::true_type{}, i);
        step(H1{}, std::true_type{}, i + 1);
    }
    // The last steps (i is even here).
    for (; i < mine; i += 2) {
        step(H0{}, std::false_type{}, i);
        if (i + 1 < mine)
            step(H1{}, std::false_type{}, i + 1);
    }

    // Sum the partial tiles of the waves in a fixed order (wave 0's first).
    // The loop above has already waited for all of this wave's ring loads.
    __syncthreads();
    float *part = lds + wave * BM * PITCH;
    const int g = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                part[(32 * i + 8 * (v >> 2) + 4 * g + (v & 3)) * PITCH + 32 * t + (lane & 31)] =
                    acc[i][t][v];

    // Epilogue: thread (wave, lane) finishes column lane % BN of rows
    // RPW * (wave + WAVES * r) + lane / BN, so every C access of a wave covers
    // whole contiguous row segments. With beta != 0 the C loads are issued
    // before the barrier and land while the partials are summed.
    const long long cbase = (long long)m0 * p.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(Cb + cbase, (long long)(p.M - 1) * p.ldc + p.N - cbase);
    const int col = lane % BN, sub = lane / BN;
    const bool col_ok = n0 + col < p.N;
    uint32_t off[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = RPW * (wave + WAVES * r) + sub;
        off[r] = (col_ok && m0 + row < p.M) ? (uint32_t)(((long long)row * p.ldc + col) * 4)
                                            : kOOB;
    }
    const bool with_beta = p.beta != 0.0f;
    float cin[RPT];
    if (with_beta) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            cin[r] = load1(rc, off[r]);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = RPW * (wave + WAVES * r) + sub;
        float x = lds[row * PITCH + col];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            x += lds[(w * BM + row) * PITCH + col];
        store1(rc, off[r], with_beta ? p.alpha * x + p.beta * cin[r] : p.alpha * x);
    }
}

// ---------------------------------------------------------------------------
// Tile kernel with direct-to-LDS staging: the tile, wave layout, LDS layout,
// fragment reads and epilogue of sgemm_mfma_kernel (WAVES_K = 1), but every
// K-step tile goes from global memory straight into LDS with buffer_load ...
// lds. Wave w issues the 1 KiB blocks w, w + NW, ... of each operand's tile,
// so no registers stage the data and no LDS write instructions are issued.
// Three LDS stages form a ring: at the start of step s the loads of step s+2
// go into the stage step s-1 occupied (every wave finished reading it before
// the barrier that ended step s-1). At the end of step s each wave waits until
// only its step s+2 loads are in flight (vector-memory operations complete in
// issue order), and the barrier then publishes step s+1 to all waves. The
// loads stop at the last step, so none is pending when the workgroup ends.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, int MIN_WAVES_PER_EU, bool A_KC, bool B_KC>
__global__ void
__attribute__((amdgpu_flat_work_group_size(64 * WAVES_M * WAVES_N, 64 * WAVES_M * WAVES_N),
               amdgpu_waves_per_eu(MIN_WAVES_PER_EU)))
sgemm_dma_kernel(Params p)
{
    constexpr int BK = 16, NW = WAVES_M * WAVES_N, NT = 64 * NW;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 32, TN = WN / 32;
    constexpr int NQ = BK / 8, LATE = TM * TN;
    using FA = Operand<A_KC, BM, BK, NT, 4>; // LDS layout and fragment reads
    using FB = Operand<B_KC, BN, BK, NT, 4>;
    using DA = DmaOperand<A_KC, BM, BK, NW>;
    using DB = DmaOperand<B_KC, BN, BK, NW>;
    static_assert(FA::STAGE == DA::FLOATS && FB::STAGE == DB::FLOATS, "one layout");
    constexpr int STAGE = FA::STAGE + FB::STAGE;
    constexpr int NI = DA::NBW + DB::NBW; // load instructions per wave and step
    static_assert(NI <= 63, "vmcnt holds at most 63");
    __shared__ __attribute__((aligned(16))) float lds[3 * STAGE];

    int b, tile_m, tile_n;
    tile_of(p, b, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave % WAVES_M) * WM, wn0 = (wave / WAVES_M) * WN;

    // K range of this workgroup, as in sgemm_mfma_kernel.
    int item = b, k0 = 0, Kt = p.K;
    if (p.splits > 1) {
        item = b / p.splits;
        k0 = (b - item * p.splits) * p.kslice;
        Kt = min(p.kslice, p.K - k0);
    }
    const float *Ab = item_a(p, item) + (A_KC ? (long long)k0 : (long long)k0 * p.lda);
    const float *Bb = item_b(p, item) + (B_KC ? (long long)k0 : (long long)k0 * p.ldb);
    float *Cb = item_c(p, b);
    if (((uintptr_t)Ab | (uintptr_t)Bb) & 15u) {
        plain_tile<BM, BN, NT, A_KC, B_KC>(p, Ab, Bb, Cb, Kt, m0, n0);
        return;
    }

    DA da;
    da.X = Ab;
    da.ld = p.lda;
    da.total = A_KC ? (long long)(p.M - 1) * p.lda + Kt : (long long)(Kt - 1) * p.lda + p.M;
    da.O = p.M;
    da.K = Kt;
    da.o0 = m0;
    // A K that is not a multiple of BK puts its partial step first, as in
    // sgemm_mfma_kernel: only the first step's loads carry a k mask.
    const int kfirst = Kt % BK == 0 ? 0 : Kt % BK - BK;
    da.init(lane, kfirst, BK, wave);
    DB db;
    db.X = Bb;
    db.ld = p.ldb;
    db.total = B_KC ? (long long)(p.N - 1) * p.ldb + Kt : (long long)(Kt - 1) * p.ldb + p.N;
    db.O = p.N;
    db.K = Kt;
    db.o0 = n0;
    db.init(lane, kfirst, BK, wave);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    const int nsteps = (Kt + BK - 1) / BK;
    auto issue = [&](float *stage, auto tail) {
        da.template issue<decltype(tail)::value>(stage, lane);
        db.template issue<decltype(tail)::value>(stage + FA::STAGE, lane);
    };
    auto read_group = [&](const float *stage, int q, float (&fa)[TM][4], float (&fb)[TN][4]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            FA::frag(stage, wm0 + 32 * i, q, lane, fa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            FB::frag(stage + FA::STAGE, wn0 + 32 * j, q, lane, fb[j]);
    };
    auto mfma_group = [&](const float (&fa)[TM][4], const float (&fb)[TN][4], int first, int last) {
#pragma unroll
        for (int t = 0; t < 4 * TM * TN; ++t) {
            if (t < first || t >= last)
                continue;
            const int kk = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk], fb[j][kk], acc[i][j],
                                                              0, 0, 0);
        }
    };

    // Steps 0 and 1 into stages 0 and 1; wait for step 0.
    issue(lds, std::true_type{});
    if (nsteps > 1) {
        issue(lds + STAGE, std::false_type{});
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NI));
    } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();
    float fa[NQ][TM][4], fb[NQ][TN][4];
    read_group(lds, 0, fa[0], fb[0]);

    // Step s in stage STG = s % 3. MODE 0 issues step s+2 (every step after
    // the first is full, so without a k mask), 2 issues nothing (s+2 is past
    // the last step).
    auto k_step = [&](auto stg, auto mode) {
        constexpr int STG = decltype(stg)::value, MODE = decltype(mode)::value;
        const float *cur = lds + STG * STAGE;
        const float *nxt = lds + ((STG + 1) % 3) * STAGE;
        float *ahead = lds + ((STG + 2) % 3) * STAGE;
        if constexpr (MODE == 0)
            issue(ahead, std::false_type{});
#pragma unroll
        for (int q = 1; q < NQ; ++q)
            read_group(cur, q, fa[q], fb[q]);
        mfma_group(fa[0], fb[0], 0, 4 * TM * TN);
#pragma unroll
        for (int q = 1; q < NQ - 1; ++q)
            mfma_group(fa[q], fb[q], 0, 4 * TM * TN);
        mfma_group(fa[NQ - 1], fb[NQ - 1], 0, 4 * TM * TN - LATE);
        // Order: the loads, this stage's remaining fragment reads, the MFMAs.
        if constexpr (MODE != 2)
            __builtin_amdgcn_sched_group_barrier(0x020, NI, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN) * (NQ - 1), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * TM * TN * NQ - LATE, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == 2)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(NI));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // (After the last step this reads a stage whose values are unused.)
        read_group(nxt, 0, fa[0], fb[0]);
        mfma_group(fa[NQ - 1], fb[NQ - 1], 4 * TM * TN - LATE, 4 * TM * TN);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (TM + TN), 0); // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, LATE, 0);          // MFMAs
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using Plain = std::integral_constant<int, 0>;
    using NoLoad = std::integral_constant<int, 2>;
    // Steps before `steady` (those with s + 2 < nsteps) issue the loads of step s + 2.
    const int steady = nsteps - 2;
    int s = 0;
    for (; s + 3 <= steady; s += 3) {
        k_step(S0{}, Plain{});
        k_step(S1{}, Plain{});
        k_step(S2{}, Plain{});
    }
    // The rest, s % 3 == 0 at entry: one copy per (stage, mode).
    auto any_step = [&](auto stg, int st) {
        if (st < steady)
            k_step(stg, Plain{});
        else
            k_step(stg, NoLoad{});
    };
    for (; s < nsteps; s += 3) {
        any_step(S0{}, s);
        if (s + 1 < nsteps)
            any_step(S1{}, s + 1);
        if (s + 2 < nsteps)
            any_step(S2{}, s + 2);
    }

    float res[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                res[i][j][v] = acc[i][j][v];
    store_tile<TM, TN, 16>(p, Cb, m0, n0, wm0, wn0, 0, lane, res);
}

// Matrix-vector product, the N == 1 case with both operands contiguous in k:
// y[m] = alpha * sum_k A[m, k] x[k] + beta * y[m], A's rows lda apart, x the K
// floats of op(B), y[m] at C[m * ldc]. It moves K floats of A per output and
// does two flops per float, far below the MFMA ridge, so it is plain FMAs at
// the HBM rate. A workgroup owns ROWS rows; its 256 threads take the 4-float
// chunks of k round-robin, keeping UNROLL chunks of every row in flight, and
// the partial sums are added across each wave with lane exchanges and across
// the four waves in LDS, always in the same order.
template <int ROWS>
__global__ void __launch_bounds__(256) sgemv_kernel(Params p)
{
    constexpr int T = 256, UNROLL = 4, WAVES = T / 64;
    const int b = blockIdx.y;
    const int m0 = p.row_base + blockIdx.x * ROWS;
    const int t = threadIdx.x;
    const float *A = item_a(p, b), *x = item_b(p, b);
    float *C = item_c(p, b);
    // Rows past M read row M - 1 again; their sums are dropped.
    const float *row[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        row[r] = A + (long long)min(m0 + r, p.M - 1) * p.lda;
    float acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        acc[r] = 0.0f;
    if (((uintptr_t)A | (uintptr_t)x) & 15u) {
        // An item of the pointer-array form off 16-byte alignment.
        for (int k = t; k < p.K; k += T) {
            const float xv = x[k];
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                acc[r] = fmaf(row[r][k], xv, acc[r]);
        }
    } else {
        const int K4 = p.K >> 2; // the host guarantees K % 4 == 0 and lda % 4 == 0
        auto dot4 = [](const f32x4 &a, const f32x4 &v, float s) {
            s = fmaf(a[0], v[0], s);
            s = fmaf(a[1], v[1], s);
            s = fmaf(a[2], v[2], s);
            return fmaf(a[3], v[3], s);
        };
        int c = t;
        for (; c + (UNROLL - 1) * T < K4; c += UNROLL * T) {
            f32x4 xv[UNROLL], av[UNROLL][ROWS];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                xv[u] = global_load4(x + 4 * (c + u * T));
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    av[u][r] = global_load4(row[r] + 4 * (c + u * T));
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    acc[r] = dot4(av[u][r], xv[u], acc[r]);
        }
        for (; c < K4; c += T) {
            const f32x4 xv = global_load4(x + 4 * c);
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                acc[r] = dot4(global_load4(row[r] + 4 * c), xv, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            acc[r] += __shfl_xor(acc[r], off);
    __shared__ float part[WAVES][ROWS];
    if ((t & 63) == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            part[t >> 6][r] = acc[r];
    }
    __syncthreads();
    if (t < ROWS && m0 + t < p.M) {
        float sum = part[0][t];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            sum += part[w][t];
        float *y = C + (long long)(m0 + t) * p.ldc;
        *y = p.beta == 0.0f ? p.alpha * sum : p.alpha * sum + p.beta * *y;
    }
}

// The same for a few vectors, 2 <= N <= NV: y[m, j] = alpha * sum_k A[m, k]
// op(B)[k, j] + beta * y[m, j], y[m, j] at C[m * ldc + j] (CT: at
// C[j * ldc + m], the product written transposed). op(B) is B's rows (B_KC: B
// stored N x K, vector j at B + j * ldb) or B stored K x N (rows of N floats
// ldb apart; N is then a multiple of 4 and NV == N). Each thread's 4-float
// chunk of k of every row meets the same four k of every vector.
template <int ROWS, int NV, bool B_KC, bool CT>
__global__ void __launch_bounds__(256) sgemv_nv_kernel(Params p)
{
    constexpr int T = 256, WAVES = T / 64;
    const int b = blockIdx.y;
    const int m0 = p.row_base + blockIdx.x * ROWS;
    const int t = threadIdx.x;
    const int N = p.N;
    const float *A = item_a(p, b), *B = item_b(p, b);
    float *C = item_c(p, b);
    // Rows past M read row M - 1 again, vectors past N vector N - 1; those
    // sums are dropped.
    const float *row[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        row[r] = A + (long long)min(m0 + r, p.M - 1) * p.lda;
    float acc[ROWS][NV];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            acc[r][j] = 0.0f;
    if (((uintptr_t)A | (uintptr_t)B) & 15u) {
        // An item of the pointer-array form off 16-byte alignment.
        for (int k = t; k < p.K; k += T) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int jj = min(j, N - 1);
                const float xv = B_KC ? B[(long long)jj * p.ldb + k] : B[(long long)k * p.ldb + jj];
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    acc[r][j] = fmaf(row[r][k], xv, acc[r][j]);
            }
        }
    } else {
        const int K4 = p.K >> 2; // the host guarantees K, lda and ldb % 4 == 0
#pragma unroll 2
        for (int c = t; c < K4; c += T) {
            float x[4][NV];
            if constexpr (B_KC) {
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const f32x4 v = global_load4(B + (long long)min(j, N - 1) * p.ldb + 4 * c);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        x[kk][j] = v[kk];
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int v = 0; v < NV / 4; ++v) {
                        const f32x4 q = global_load4(B + (long long)(4 * c + kk) * p.ldb + 4 * v);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[kk][4 * v + e] = q[e];
                    }
            }
            f32x4 av[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                av[r] = global_load4(row[r] + 4 * c);
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acc[r][j] = fmaf(av[r][kk], x[kk][j], acc[r][j]);
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                acc[r][j] += __shfl_xor(acc[r][j], off);
    __shared__ float part[WAVES][ROWS][NV];
    if ((t & 63) == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int j = 0; j < NV; ++j)
                part[t >> 6][r][j] = acc[r][j];
    }
    __syncthreads();
    if (t < ROWS * NV) {
        const int r = t / NV, j = t % NV;
        if (m0 + r < p.M && j < N) {
            float sum = part[0][r][j];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                sum += part[w][r][j];
            float *y = CT ? C + (long long)j * p.ldc + (m0 + r) : C + (long long)(m0 + r) * p.ldc + j;
            *y = p.beta == 0.0f ? p.alpha * sum : p.alpha * sum + p.beta * *y;
        }
    }
}

// Matrix-vector product with the matrix contiguous along the outputs, the
// N == 1 case with A stored K x M: y[m] = alpha * sum_k A[k * lda + m] x[k] +
// beta * y[m], x the K floats of op(B), y[m] at C[m * ldc]. A workgroup owns
// BC outputs. A load instruction of a wave covers RPI = 256 / BC consecutive
// rows, BC / 4 lanes of 16 bytes per row; the eight waves take turns of RPI
// rows each, UNROLL loads in flight. The partial sums are added across the
// lanes of a column group, then across the waves in LDS, in a fixed order.
template <int BC>
__global__ void __launch_bounds__(512) sgemv_t_kernel(Params p)
{
    constexpr int WAVES = 8, LPR = BC / 4, RPI = 64 / LPR, UNROLL = 8, STEP = WAVES * RPI;
    const int b = blockIdx.y;
    // Neighbouring column blocks share 128-byte lines: each XCD (workgroup
    // pid runs on XCD pid % 8) gets a contiguous range of blocks.
    const int num = gridDim.x, pid = blockIdx.x;
    const int xcd = pid % kNumXcd, local = pid / kNumXcd;
    const int q = num / kNumXcd, r = num % kNumXcd;
    const int blk = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    const int m0 = p.row_base + blk * BC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane % LPR, ro = lane / LPR;
    const int m = m0 + 4 * cg; // the host guarantees M % 4 == 0 and lda % 4 == 0
    const float *A = item_a(p, b), *x = item_b(p, b);
    float *C = item_c(p, b);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (m < p.M) {
        const float *col = A + m;
        int k = wave * RPI + ro;
        if (((uintptr_t)A | (uintptr_t)x) & 15u) {
            // An item of the pointer-array form off 16-byte alignment.
            for (; k < p.K; k += STEP) {
                const float xv = x[k];
                const float *a = col + (long long)k * p.lda;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j] = fmaf(a[j], xv, acc[j]);
            }
        } else {
            const int kfull = p.K - (UNROLL - 1) * STEP; // k < kfull: all UNROLL rows exist
            for (; k < kfull; k += UNROLL * STEP) {
                f32x4 av[UNROLL];
                float xv[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    av[u] = global_load4(col + (long long)(k + u * STEP) * p.lda);
                    xv[u] = global_load1(x + k + u * STEP);
                }
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[j] = fmaf(av[u][j], xv[u], acc[j]);
            }
            for (; k < p.K; k += STEP) {
                const f32x4 av = global_load4(col + (long long)k * p.lda);
                const float xv = global_load1(x + k);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j] = fmaf(av[j], xv, acc[j]);
            }
        }
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j] += __shfl_xor(acc[j], off);
    __shared__ f32x4 part[WAVES][LPR];
    if (ro == 0)
        part[wave][cg] = acc;
    __syncthreads();
    const int t = threadIdx.x;
    if (t < LPR && m0 + 4 * t < p.M) {
        f32x4 sum = part[0][t];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            sum += part[w][t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float *y = C + (long long)(m0 + 4 * t + j) * p.ldc;
            *y = p.beta == 0.0f ? p.alpha * sum[j] : p.alpha * sum[j] + p.beta * *y;
        }
    }
}

// C = beta * C over the M x N window of every batch item (alpha == 0 or K == 0).
__global__ void __launch_bounds__(256) sgemm_scale_kernel(float *C, float *const *Carr, int M,
                                                          int N, int ldc, long long sC,
                                                          int batch, float beta)
{
    const long long per = (long long)M * N;
    const long long total = per * batch;
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total;
         e += (long long)gridDim.x * 256) {
        const long long b = e / per, r = (e % per) / N, c = e % N;
        float *x = (Carr ? Carr[b] : C + b * sC) + r * ldc + c;
        *x = beta == 0.0f ? 0.0f : beta * *x;
    }
}

// Split-K epilogue: C = alpha * (sum of the item's partial tiles, slice 0
// first) + beta * C over the M x N window of every batch item. W holds the
// partials of item i, slice s at W + (i * splits + s) * M * N, rows of N.
// The summation order is fixed, so results do not depend on timing.
__global__ void __launch_bounds__(256) sgemm_splitk_reduce_kernel(const float *W, float *C,
                                                                  float *const *Carr, int M,
                                                                  int N, int ldc, long long sC,
                                                                  int items, int splits,
                                                                  float alpha, float beta)
{
    const long long per = (long long)M * N;
    const long long total = per * items;
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total;
         e += (long long)gridDim.x * 256) {
        const long long item = e / per, in_item = e - item * per;
        const long long r = in_item / N, c = in_item - r * N;
        const float *w = W + item * splits * per + in_item;
        float sum = w[0];
        for (int sl = 1; sl < splits; ++sl)
            sum += w[sl * per];
        float *x = (Carr ? Carr[item] : C + item * sC) + r * ldc + c;
        *x = beta == 0.0f ? alpha * sum : alpha * sum + beta * *x;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

typedef void (*KernelFn)(Params);

struct VariantInfo {
    int bm, bn, bk, threads, vec;
    KernelFn fn[2][2]; // [transA][transB]; every kernel takes any K
};

constexpr int kBK = 16;

template <int BM, int BN, int BK, int WM_, int WN_, int WK_, int MW, int VEC, bool WIDE = false>
constexpr VariantInfo make_variant()
{
    return VariantInfo{BM, BN, BK, 64 * WM_ * WN_ * WK_, VEC,
                       {{sgemm_mfma_kernel<BM, BN, BK, WM_, WN_, WK_, MW, true, false, VEC, WIDE>,
                         sgemm_mfma_kernel<BM, BN, BK, WM_, WN_, WK_, MW, true, true, VEC, WIDE>},
                        {sgemm_mfma_kernel<BM, BN, BK, WM_, WN_, WK_, MW, false, false, VEC, WIDE>,
                         sgemm_mfma_kernel<BM, BN, BK, WM_, WN_, WK_, MW, false, true, VEC, WIDE>}}};
}

template <int BM, int BN, int WM_, int WN_, int MW>
constexpr VariantInfo make_dma_variant()
{
    return VariantInfo{BM, BN, 16, 64 * WM_ * WN_, 4,
                       {{sgemm_dma_kernel<BM, BN, WM_, WN_, MW, true, false>,
                         sgemm_dma_kernel<BM, BN, WM_, WN_, MW, true, true>},
                        {sgemm_dma_kernel<BM, BN, WM_, WN_, MW, false, false>,
                         sgemm_dma_kernel<BM, BN, WM_, WN_, MW, false, true>}}};
}

template <int BM, int BN>
constexpr VariantInfo make_persistent_variant()
{
    return VariantInfo{BM, BN, 16, 768, 4,
                       {{sgemm_persistent_kernel<BM, BN, true, false>,
                         sgemm_persistent_kernel<BM, BN, true, true>},
                        {sgemm_persistent_kernel<BM, BN, false, false>,
                         sgemm_persistent_kernel<BM, BN, false, true>}}};
}

template <int WAVES, int STAGES, int BM, int BN, int MINW>
constexpr VariantInfo make_stream_variant()
{
    return VariantInfo{BM, BN, 16, 64 * WAVES, 4,
                       {{sgemm_stream_kernel<WAVES, STAGES, BM, BN, MINW, true, false>,
                         sgemm_stream_kernel<WAVES, STAGES, BM, BN, MINW, true, true>},
                        {sgemm_stream_kernel<WAVES, STAGES, BM, BN, MINW, false, false>,
                         sgemm_stream_kernel<WAVES, STAGES, BM, BN, MINW, false, true>}}};
}

const VariantInfo kVariants[SGEMM_VARIANT_COUNT] = {
    make_variant<256, 128, kBK, 2, 2, 1, 2, 4>(), // SGEMM_VARIANT_L256x128
    make_variant<128, 128, kBK, 2, 2, 1, 2, 4>(), // SGEMM_VARIANT_M128x128
    make_variant<64, 64, kBK, 2, 2, 1, 4, 4>(),   // SGEMM_VARIANT_S64x64
    make_variant<64, 64, kBK, 2, 2, 1, 4, 1>(),   // SGEMM_VARIANT_S64x64_V1
    make_stream_variant<4, 4, 64, 64, 1>(),       // SGEMM_VARIANT_T64x64
    make_variant<256, 256, kBK, 2, 4, 1, 2, 4>(), // SGEMM_VARIANT_L256x256
    make_variant<64, 64, 32, 2, 2, 2, 2, 4>(),    // SGEMM_VARIANT_S64x64_K2
    make_dma_variant<128, 128, 2, 2, 2>(),        // SGEMM_VARIANT_M128x128_DMA
    make_stream_variant<8, 3, 32, 64, 2>(),       // SGEMM_VARIANT_T32x64
    make_stream_variant<8, 3, 64, 32, 2>(),       // SGEMM_VARIANT_T64x32
    // SGEMM_VARIANT_GEMV: N == 1 (or M == 1, as its transpose) with the vector
    // contiguous in k; launched by launch_gemv, which picks the kernel.
    VariantInfo{4, 1, 4, 256, 4, {{nullptr, sgemv_kernel<4>}, {nullptr, sgemv_t_kernel<64>}}},
    make_variant<64, 64, kBK, 2, 2, 1, 4, 4, true>(), // SGEMM_VARIANT_W64x64
    make_variant<64, 64, kBK, 2, 2, 1, 4, 1, true>(), // SGEMM_VARIANT_W64x64_V1
    make_persistent_variant<128, 128>(),              // SGEMM_VARIANT_P128x128
    make_persistent_variant<64, 64>(),                // SGEMM_VARIANT_P64x64
};

bool is_persistent(int variant)
{
    return variant == SGEMM_VARIANT_P128x128 || variant == SGEMM_VARIANT_P64x64;
}

// Tiles per workgroup of the persistent kernel for this grid on `cus`
// compute units (one workgroup each), or 0 when it cannot run it: the tiles
// must split evenly over the workgroups, eight XCDs apart, into n per
// workgroup with n % 3 != 2 (its three wave groups then take whole tiles, or
// whole tiles and a third of the K range of one more each, which needs
// K >= 192 so that every third is at least four K-steps).
long long persistent_tiles(int variant, int M, int N, int K, int batch, long long cus)
{
    const VariantInfo &vi = kVariants[variant];
    const long long tiles = ((long long)M + vi.bm - 1) / vi.bm * (((long long)N + vi.bn - 1) / vi.bn) * batch;
    if (cus < 8 || cus % 8 != 0 || tiles % cus != 0 || tiles / cus > INT32_MAX || tiles > INT32_MAX)
        return 0;
    const long long n = tiles / cus;
    if (n % 3 == 2 || (n % 3 == 1 && K < 192))
        return 0;
    return n;
}

// The 64-bit-addressed builds, which take any leading dimension.
bool is_wide(int variant)
{
    return variant == SGEMM_VARIANT_W64x64 || variant == SGEMM_VARIANT_W64x64_V1;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The streaming kernels split K across their own waves and never across
// workgroups.
bool is_stream(int variant)
{
    return variant == SGEMM_VARIANT_T64x64 || variant == SGEMM_VARIANT_T32x64 ||
           variant == SGEMM_VARIANT_T64x32;
}

// Variants that never split K across workgroups.
bool no_split(int variant)
{
    return is_stream(variant) || variant == SGEMM_VARIANT_GEMV || is_persistent(variant);
}

int num_cus_of_current_device(int *out)
{
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev >= 0 && dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) {
            *out = v;
            return 0;
        }
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev >= 0 && dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return 0;
}

int validate(int tA, int tB, int M, int N, int K, const float *A, int lda, const float *B,
             int ldb, const float *C, int ldc, int batch, long long sA, long long sB,
             long long sC, float alpha, float beta)
{
    if (tA != 0 && tA != 1) return -1;
    if (tB != 0 && tB != 1) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    const int rowA = tA ? M : K, rowB = tB ? K : N;
    if (lda < (rowA > 1 ? rowA : 1)) return -8;
    if (ldb < (rowB > 1 ? rowB : 1)) return -10;
    if (ldc < (N > 1 ? N : 1)) return -13;
    if (batch < 0) return -14;
    if (sA < 0) return -15;
    if (sB < 0) return -16;
    if (sC < 0) return -17;
    const bool work = M > 0 && N > 0 && batch > 0;
    const bool product = work && K > 0 && alpha != 0.0f;
    const bool touch_c = work && (product || beta != 1.0f);
    if (product && A == nullptr) return -7;
    if (product && B == nullptr) return -9;
    if (touch_c && C == nullptr) return -12;
    return 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Per-shape dispatch overrides: exact call shapes and the variant the
// automatic choice takes for each, installed by the caller from an offline
// sweep. Every automatic choice looks its shape up, so with no table
// installed the lookup is one atomic load.
struct ShapeKey {
    int tA, tB, M, N, K, batch;
    bool operator==(const ShapeKey &o) const
    {
        return tA == o.tA && tB == o.tB && M == o.M && N == o.N && K == o.K && batch == o.batch;
    }
};
struct ShapeHash {
    size_t operator()(const ShapeKey &k) const
    {
        uint64_t h = 0x9e3779b97f4a7c15ull;
        for (const int v : {k.tA, k.tB, k.M, k.N, k.K, k.batch})
            h = (h ^ (uint32_t)v) * 0x100000001b3ull;
        return (size_t)h;
    }
};
using OverrideTable = std::unordered_map<ShapeKey, int, ShapeHash>;
std::shared_mutex g_override_mutex;
OverrideTable g_overrides;
std::atomic<int> g_override_count{0};

// Variants an override may name: those that run any shape (the tiles, the
// streaming tiles and the 64-bit-addressed tiles), not the matrix-vector or
// persistent kernels, which take only some.
bool overridable(int v)
{
    return v >= 0 && v < SGEMM_VARIANT_COUNT && v != SGEMM_VARIANT_GEMV && !is_persistent(v);
}

// The override for this shape, or -1.
int override_for(int tA, int tB, int M, int N, int K, int batch)
{
    if (g_override_count.load(std::memory_order_acquire) == 0)
        return -1;
    std::shared_lock<std::shared_mutex> lock(g_override_mutex);
    const auto it = g_overrides.find(ShapeKey{tA, tB, M, N, K, batch});
    return it == g_overrides.end() ? -1 : it->second;
}

} // namespace

extern "C" int sgemm_set_dispatch_overrides(const int *entries, int count)
{
    if (count < 0 || count > SGEMM_MAX_DISPATCH_OVERRIDES)
        return -25;
    if (count > 0 && entries == nullptr)
        return -24;
    OverrideTable table;
    table.reserve((size_t)count);
    for (int i = 0; i < count; ++i) {
        const int *e = entries + 7 * i;
        if ((e[0] != 0 && e[0] != 1) || (e[1] != 0 && e[1] != 1) || e[2] < 0 || e[3] < 0 ||
            e[4] < 0 || e[5] < 0 || !overridable(e[6]))
            return -24;
        table[ShapeKey{e[0], e[1], e[2], e[3], e[4], e[5]}] = e[6]; // a later record wins
    }
    // (the previous table is freed after the lock is released)
    std::unique_lock<std::shared_mutex> lock(g_override_mutex);
    g_overrides.swap(table);
    g_override_count.store((int)g_overrides.size(), std::memory_order_release);
    return 0;
}

extern "C" int sgemm_dispatch_override_count(void)
{
    return g_override_count.load(std::memory_order_acquire);
}

extern "C" int sgemm_select_variant(int transA, int transB, int M, int N, int K, int batch,
                                    int vec4_ok, int num_cus)
{
    if (transA != 0 && transA != 1) return -1;
    if (transB != 0 && transB != 1) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    if (batch < 0) return -14;
    // An installed override for exactly this shape, where the call's
    // alignment allows its load width.
    const int ov = override_for(transA, transB, M, N, K, batch);
    if (ov >= 0 && (vec4_ok || kVariants[ov].vec == 1))
        return ov;
    if (!vec4_ok)
        return SGEMM_VARIANT_S64x64_V1;
    // A matrix-vector product (N == 1, or M == 1 as its transpose) whose
    // vector is contiguous in k: the GEMV kernels, which stream the matrix
    // without the 32 columns of MFMA work a tile would do per output
    // (4096 x 1 x 4096: 34 µs on the 64 x 32 tile, whose 64 workgroups leave
    // most CUs idle, against 11 µs).
    if ((N == 1 && transB == 1) || (M == 1 && transA == 0))
        return SGEMM_VARIANT_GEMV;
    if (num_cus < 1)
        num_cus = 1;
    const long long cus = num_cus;
    // A few vectors (2 <= N <= 8) against a matrix contiguous in k, over a K
    // deep enough for the threads of a workgroup to share: the same kernel
    // with every 4-float chunk of A meeting the vectors' four k. Every
    // workgroup reads all the vectors, so it pays where they are few and
    // contiguous (B transposed, N <= 4: 16384 x 2 x 4096 38 against 44 µs)
    // or where the 64 x 32 tiles would not fill the CUs (4096 x 8 x 4096:
    // 27 against 34 µs); on a full grid of those tiles with B stored K x N or
    // eight vectors the tiles win (16384 x 8 x 4096: 45 against 106 µs).
    if (N >= 2 && N <= 8 && transA == 0 && K >= 512 &&
        ((transB == 1 && N <= 4) || ceil_div(M, 64) * batch < cus))
        return SGEMM_VARIANT_GEMV;
    // The mirror: a few rows (2 <= M <= 8) against B stored N x K, run as the
    // transpose with C^T written transposed (Y = X W^T with X a handful of
    // rows and W stored N x K).
    if (M >= 2 && M <= 8 && transB == 1 && K >= 512 &&
        ((transA == 0 && M <= 4) || ceil_div(N, 64) * batch < cus))
        return SGEMM_VARIANT_GEMV;
    const long long tiles64 = ceil_div(M, 64) * ceil_div(N, 64) * batch;
    const long long tiles32 = ceil_div(M, 32) * ceil_div(N, 64) * batch;
    const long long tiles6432 = ceil_div(M, 64) * ceil_div(N, 32) * batch;
    // The eight-wave streaming kernel on a 64 x 32 or 32 x 64 tile: with at
    // most one such tile per CU a call takes as long as one workgroup's tile,
    // which is half a 64 x 64 tile with two waves per SIMD on it (8192 x 64 x
    // 4096: 37 µs against 59 µs for the K-split 64 x 64 tile; 512 x 512 x 384:
    // 7.0 against 8.7 µs; 128^3: 5.3 against 6.0 µs). Over K >= 512 the 64 x 32
    // tile is 2-5 % faster than the 32 x 64 one (512^3: 7.7 against 8.1 µs;
    // 640 x 480 x 2000: 19.5 against 20.0 µs); below, the 32 x 64 tile is
    // (128^3: 5.1 against 5.3 µs). With a single row (M <= 32) or column
    // (N <= 32) of tiles over a deep K the matching tile is also the best for
    // any number of them: the 64 x 64 tiles come in the same number and each
    // takes longer (16384 x 1 x 4096: 44 µs against 64 µs).
    const bool few6432 = tiles6432 <= cus;
    if (M > 32 && (N <= 32 ? few6432 || K >= 512 : few6432 && K >= 512))
        return SGEMM_VARIANT_T64x32;
    if (tiles32 <= cus || (M <= 32 && K >= 512))
        return SGEMM_VARIANT_T32x64;
    // One skinny dimension (<= 64) over a deep K, one 64 x 64 tile per CU at
    // most, a long operand contiguous in k and too large to stay in the
    // 256 MB Infinity Cache from one call to the next (over 128 MiB), and the
    // short operand contiguous along its outputs: the four-wave 64 x 64
    // streaming kernel, whose 4-deep per-wave rings stream that operand from
    // HBM faster than the K-split tile does in this layout (16384 x 64 x 4096
    // NN with operands from HBM: 78.5 against 83.9 µs; 16384 x 64 x 8192 NN:
    // 149.6 against 167.7 µs; 64 x 16384 x 4096 TT: 77.6 against 80.2 µs).
    // In the other layouts, with two tiles per CU, or with a long operand
    // that stays cached, the K-split tile below is as fast or faster
    // (16384 x 64 x 4096 NT: 78.1 against 79.3 µs; TT 74.0 against 76.6 µs;
    // 32768 x 64 x 4096 NN: 148.3 against 152.3 µs).
    const bool long_a = M > N;
    const long long long_bytes = 4LL * (long_a ? M : N) * K * batch;
    const bool long_kc = long_a ? transA == 0 : transB == 1;
    const bool short_outer = long_a ? transB == 0 : transA == 1;
    if ((M <= 64 || N <= 64) && K >= 512 && tiles64 <= cus && long_kc && short_outer &&
        long_bytes > (128LL << 20))
        return SGEMM_VARIANT_T64x64;
    // Otherwise the tile whose busiest CU finishes first: a CU receives
    // ceil(tiles / CUs) tiles, each costing its area over the variant's
    // relative efficiency. The efficiencies are fitted to sweeps of every
    // variant over 76 shapes (precision_gemm_amd/tune.py): 128 x 128 tiles
    // 1.00; the K-split 64 x 64 tile 0.88, for K >= 768; plain 64 x 64 tiles
    // 0.85, or 1.05 for K <= 128, where a tile's fixed costs (the first loads,
    // the C stores) outweigh its short K loop and the small tiles, more of
    // them resident per CU, overlap those costs better (8192^2 x 128: 185 µs
    // against 193; 2048^2 x 64: 10.1 against 10.7), and 0.99 for 128 < K <=
    // 512, where the 128 x 128 tile wins an equal share of work per CU
    // (4096^2 x 256: 70.7 against 75.4 µs; 256^3 x 128 items: 37.4 against
    // 38.8) and loses only where it would leave CUs idle; the streaming 64 x 32
    // tile 0.78, for K >= 2048 (any value from 0.75 to 0.80 picks the same
    // variants on the sweeps), whose small area fills the last round of tiles
    // better (1152^2 x 4096: 100 µs against 118 µs for the K-split tile). The
    // 256-row tiles and the direct-to-LDS 128 x 128 tile never won by more than
    // the sweeps' noise on the shapes that matter, so they are left to
    // explicit requests.
    // A tile whose grid would not fit one launch (more than 2^31 - 1
    // work-items per item along the tile axis) is skipped.
    struct Choice { int variant, bm, bn, eff_pct; long long min_k; };
    const Choice choices[] = {{SGEMM_VARIANT_M128x128, 128, 128, 100, 0},
                              {SGEMM_VARIANT_S64x64_K2, 64, 64, 88, 768},
                              {SGEMM_VARIANT_S64x64, 64, 64, K <= 128 ? 105 : K <= 512 ? 99 : 85, 0},
                              {SGEMM_VARIANT_T64x32, 64, 32, 78, 2048}};
    int best = SGEMM_VARIANT_M128x128;
    double best_cost = -1.0;
    for (const Choice &c : choices) {
        if (K < c.min_k ||
            ceil_div(M, c.bm) * ceil_div(N, c.bn) * kVariants[c.variant].threads > INT32_MAX)
            continue;
        const long long tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn) * batch;
        const double cost = (double)ceil_div(tiles, cus) * c.bm * c.bn * 100.0 / c.eff_pct;
        if (best_cost < 0 || cost < best_cost) {
            best = c.variant;
            best_cost = cost;
        }
    }
    return best;
}

namespace {

constexpr int kMinSliceK = 256; // shortest K slice worth a workgroup of its own
constexpr int kSliceCostK = 256; // a workgroup's fixed cost (pipeline fill, epilogue) in k
constexpr int kMaxSplits = 128;

// Split count for `variant` (a tile kernel): the S that minimises the busiest
// CU's work, ceil(tiles * S / CUs) workgroups of (K / S + kSliceCostK) k each,
// over slices at least kMinSliceK deep and at most kMaxSplits of them. A
// slice is round_up(ceil(K / S), BK) long, so the returned count is that of
// the non-empty slices; 1 means no split.
long long splits_for(int variant, int M, int N, int K, int batch, long long cus, int *kslice)
{
    const VariantInfo &vi = kVariants[variant];
    *kslice = K;
    if (M == 0 || N == 0 || K == 0 || batch == 0)
        return 1;
    const long long tiles = ceil_div(M, vi.bm) * ceil_div(N, vi.bn) * batch;
    long long smax = K / kMinSliceK;
    if (smax > kMaxSplits)
        smax = kMaxSplits;
    long long best_s = 1, best_ks = K;
    long long best_cost = ceil_div(tiles, cus) * ((long long)K + kSliceCostK);
    for (long long S = 2; S <= smax; ++S) {
        const long long ks = ceil_div(ceil_div(K, S), vi.bk) * vi.bk;
        const long long se = ceil_div(K, ks);
        const long long cost = ceil_div(tiles * se, cus) * (ks + kSliceCostK);
        if (cost < best_cost) {
            best_cost = cost;
            best_s = se;
            best_ks = ks;
        }
    }
    *kslice = (int)best_ks;
    return best_s;
}

} // namespace

extern "C" int sgemm_select_splits(int transA, int transB, int M, int N, int K, int batch,
                                   int variant, int num_cus)
{
    if (transA != 0 && transA != 1) return -1;
    if (transB != 0 && transB != 1) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    if (batch < 0) return -14;
    if (variant < 0 || variant >= SGEMM_VARIANT_COUNT)
        return -18;
    if (no_split(variant))
        return 1;
    int kslice = 0;
    return (int)splits_for(variant, M, N, K, batch, num_cus < 1 ? 1 : num_cus, &kslice);
}

namespace {

// One validated call in row-major terms. Either the strided bases (A, B, C
// with sA, sB, sC) or the pointer arrays (Aarr, Barr, Carr) describe the
// batch items.
struct Call {
    int tA, tB, M, N, K;
    float alpha, beta;
    const float *A, *B;
    float *C;
    int lda, ldb, ldc, batch;
    long long sA, sB, sC;
    const float *const *Aarr;
    const float *const *Barr;
    float *const *Carr;
};

// Workspace of a split-K call: `ws` (4-byte aligned, or NULL) of `ws_bytes`.
// splits: 0 = choose (only with a workspace), 1 = none, >= 2 forced.
struct Split {
    float *ws;
    size_t ws_bytes;
    int splits;
};

int launch_canonical(const Call &c, int variant, hipStream_t s, Split sk);

int launch(const Call &c, int variant, hipStream_t s, Split sk = Split{nullptr, 0, 1})
{
    if (c.M == 0 || c.N == 0 || c.batch == 0)
        return 0;
    if (c.K == 0 || c.alpha == 0.0f) {
        if (c.beta == 1.0f)
            return 0;
        const long long total = (long long)c.M * c.N * c.batch;
        const long long blocks = ceil_div(total, 256) < 8192 ? ceil_div(total, 256) : 8192;
        float *C = c.C;
        float *const *Carr = c.Carr;
        int M = c.M, N = c.N, ldc = c.ldc, batch = c.batch;
        long long sC = c.sC;
        float beta = c.beta;
        void *args[] = {&C, &Carr, &M, &N, &ldc, &sC, &batch, &beta};
        return (int)hipLaunchKernel((const void *)sgemm_scale_kernel, dim3((unsigned)blocks),
                                    dim3(256), args, 0, s);
    }

    // A vector operand (M == 1 or N == 1) whose K elements are contiguous is
    // the same memory in the k-contiguous description: op(B) with N == 1,
    // transB == 0 and ldb == 1 is B[k], as with transB == 1 and any ldb >= K
    // (likewise op(A) with M == 1, transA == 1, lda == 1). That description
    // allows the 16-byte loads along k.
    Call cc = c;
    if (cc.N == 1 && cc.tB == 0 && cc.ldb == 1 && cc.K > 1) {
        cc.tB = 1;
        cc.ldb = cc.K;
    }
    if (cc.M == 1 && cc.tA == 1 && cc.lda == 1 && cc.K > 1) {
        cc.tA = 0;
        cc.lda = cc.K;
    }
    return launch_canonical(cc, variant, s, sk);
}

// The GEMV kernels over every batch item of an N == 1 call whose op(B) is
// contiguous in k (op(A) contiguous in k, transA == 0, or along M), or of a
// call with 2 <= N <= 8 and op(A) contiguous in k (op(B) either way);
// c_transposed: the product goes to C transposed (C^T of the caller's call).
int launch_gemv(const Call &c, hipStream_t s, bool c_transposed)
{
    int cus = 0;
    const int st = num_cus_of_current_device(&cus);
    if (st != 0)
        return st;
    long long blocks;
    int threads, rows_per_block;
    KernelFn fn;
    if (c.N > 1) {
        // A few vectors (2 <= N <= 8, A contiguous in k): four rows per
        // workgroup, or one on small grids, as for one vector.
        const bool four = ceil_div(c.M, 4) * c.batch >= 2LL * cus;
        const int nv = c.N <= 2 ? 2 : c.N <= 4 ? 4 : 8;
        static const KernelFn kc[2][2][3] = {
            {{sgemv_nv_kernel<1, 2, true, false>, sgemv_nv_kernel<1, 4, true, false>,
              sgemv_nv_kernel<1, 8, true, false>},
             {sgemv_nv_kernel<4, 2, true, false>, sgemv_nv_kernel<4, 4, true, false>,
              sgemv_nv_kernel<4, 8, true, false>}},
            {{sgemv_nv_kernel<1, 2, true, true>, sgemv_nv_kernel<1, 4, true, true>,
              sgemv_nv_kernel<1, 8, true, true>},
             {sgemv_nv_kernel<4, 2, true, true>, sgemv_nv_kernel<4, 4, true, true>,
              sgemv_nv_kernel<4, 8, true, true>}}};
        static const KernelFn kn[2][2][2] = {
            {{sgemv_nv_kernel<1, 4, false, false>, sgemv_nv_kernel<1, 8, false, false>},
             {sgemv_nv_kernel<4, 4, false, false>, sgemv_nv_kernel<4, 8, false, false>}},
            {{sgemv_nv_kernel<1, 4, false, true>, sgemv_nv_kernel<1, 8, false, true>},
             {sgemv_nv_kernel<4, 4, false, true>, sgemv_nv_kernel<4, 8, false, true>}}};
        // (B stored K x N: the host guarantees N % 4 == 0, so nv == N.)
        fn = c.tB == 1 ? kc[c_transposed][four][nv == 2 ? 0 : nv == 4 ? 1 : 2]
                       : kn[c_transposed][four][nv == 4 ? 0 : 1];
        rows_per_block = four ? 4 : 1;
        blocks = ceil_div(c.M, rows_per_block);
        threads = 256;
    } else if (c.tA == 0) {
        // Four rows per workgroup, or one when that leaves fewer than two
        // workgroups per CU.
        const int rows = ceil_div(c.M, 4) * c.batch >= 2LL * cus ? 4 : 1;
        rows_per_block = rows;
        blocks = ceil_div(c.M, rows);
        threads = 256;
        fn = rows == 4 ? sgemv_kernel<4> : sgemv_kernel<1>;
    } else {
        // The widest block of outputs (64, 32, 16 or 8: row segments of 256,
        // 128, 64 or 32 bytes) that still gives every CU a workgroup
        // (16384 x 1 x 4096: 38 µs with 64, 44 with 32, 50 with 16; 8192 x 1 x
        // 8192: 42, 40, 48 µs; 4096 x 1 x 4096: 20, 15, 14 µs; 2048 x 1 x
        // 16384: 35 µs with 16, 32 with 8). Below that 8, or 4 (16-byte
        // segments) over K >= 16384, where a deep K leaves the few workgroups
        // the whole call (1024 x 1 x 65536: 131, 109, 96 µs with 16, 8, 4;
        // 512 x 1 x 8192: 6.9 µs with 8, 8.2 with 4).
        const int bc = ceil_div(c.M, 64) * c.batch >= cus                    ? 64
                       : ceil_div(c.M, 32) * c.batch >= cus                  ? 32
                       : ceil_div(c.M, 16) * c.batch >= cus                  ? 16
                       : ceil_div(c.M, 8) * c.batch >= cus || c.K < 16384 ? 8
                                                                             : 4;
        rows_per_block = bc;
        blocks = ceil_div(c.M, bc);
        threads = 512;
        static const KernelFn kt[5] = {sgemv_t_kernel<4>, sgemv_t_kernel<8>, sgemv_t_kernel<16>,
                                       sgemv_t_kernel<32>, sgemv_t_kernel<64>};
        fn = kt[bc == 4 ? 0 : bc == 8 ? 1 : bc == 16 ? 2 : bc == 32 ? 3 : 4];
    }
    Params p{};
    p.A = c.A;
    p.B = c.B;
    p.C = c.C;
    p.Aarr = c.Aarr;
    p.Barr = c.Barr;
    p.Carr = c.Carr;
    p.M = c.M;
    p.N = c.N;
    p.K = c.K;
    p.lda = c.lda;
    p.ldb = c.ldb;
    p.ldc = c.ldc;
    p.sA = c.sA;
    p.sB = c.sB;
    p.sC = c.sC;
    p.alpha = c.alpha;
    p.beta = c.beta;
    p.tiles_m = (int)blocks;
    p.tiles_n = 1;
    p.group_m = 1;
    p.splits = 1;
    p.kslice = c.K;
    const bool arrays = c.Aarr != nullptr;
    // A launch holds at most 2^31 - 1 work-items along grid x: a taller
    // matrix runs as several launches over consecutive row blocks, each told
    // its first row (the kernels keep M itself for the bounds).
    const long long max_blocks = INT32_MAX / threads;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        const long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        for (long long k0 = 0; k0 < blocks; k0 += max_blocks) {
            const long long nk = blocks - k0 < max_blocks ? blocks - k0 : max_blocks;
            Params q = p;
            q.row_base = (int)(k0 * rows_per_block);
            if (arrays) {
                q.Aarr = c.Aarr + b0;
                q.Barr = c.Barr + b0;
                q.Carr = c.Carr + b0;
            } else {
                q.A = c.A + b0 * c.sA;
                q.B = c.B + b0 * c.sB;
                q.C = c.C + b0 * c.sC;
            }
            void *args[] = {&q};
            hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)nk, (unsigned)nb),
                                           dim3(threads), args, 0, s);
            if (e != hipSuccess)
                return (int)e;
        }
    }
    return 0;
}

int launch_canonical(const Call &c, int variant, hipStream_t s, Split sk)
{
    // 16-byte loads need aligned bases, ld and batch strides, and whole
    // 4-float chunks along each operand's contiguous dimension. Item pointers
    // of the pointer-array form are not visible here; the kernels check them.
    const bool arrays = c.Aarr != nullptr;
    const bool a_kc = c.tA == 0, b_kc = c.tB == 1;
    const bool vec4_ok =
        (arrays || (aligned16(c.A) && aligned16(c.B) && c.sA % 4 == 0 && c.sB % 4 == 0)) &&
        c.lda % 4 == 0 && c.ldb % 4 == 0 && (a_kc ? c.K % 4 == 0 : c.M % 4 == 0) &&
        (b_kc ? c.K % 4 == 0 : c.N % 4 == 0);
    const bool auto_variant = variant == SGEMM_VARIANT_AUTO;
    int cus = 0;
    if (auto_variant || sk.splits == 0 || is_persistent(variant)) {
        const int st = num_cus_of_current_device(&cus);
        if (st != 0)
            return st;
    }
    // A leading dimension beyond kMaxLd overflows the 32-bit in-tile offsets
    // of every kernel but the 64-bit-addressed tile and the GEMV kernels
    // (which address with 64-bit arithmetic throughout).
    const bool wide = c.lda > kMaxLd || c.ldb > kMaxLd || c.ldc > kMaxLd;
    if (auto_variant) {
        variant = sgemm_select_variant(c.tA, c.tB, c.M, c.N, c.K, c.batch, vec4_ok ? 1 : 0, cus);
        if (variant < 0)
            return variant;
        if (wide && variant != SGEMM_VARIANT_GEMV)
            variant = vec4_ok ? SGEMM_VARIANT_W64x64 : SGEMM_VARIANT_W64x64_V1;
    } else if ((kVariants[variant].vec == 4 && !vec4_ok) ||
               (wide && !is_wide(variant) && variant != SGEMM_VARIANT_GEMV) ||
               (is_persistent(variant) &&
                (arrays || persistent_tiles(variant, c.M, c.N, c.K, c.batch, cus) == 0))) {
        return -18;
    }
    if (variant == SGEMM_VARIANT_GEMV) {
        const bool direct = (c.N == 1 && c.tB == 1) || (c.N >= 2 && c.N <= 8 && c.tA == 0);
        const bool mirror = (c.M == 1 && c.tA == 0) || (c.M >= 2 && c.M <= 8 && c.tB == 1);
        if (!direct && !mirror)
            return -18;
        if (sk.splits >= 2)
            return -19;
        if (direct)
            return launch_gemv(c, s, false);
        // M <= 8: the transpose, C^T = op(B)^T op(A)^T, whose matrix is op(B)^T
        // (B with the other transpose flag) and whose vectors are op(A)'s rows;
        // C^T is N x 1 with rows 1 apart for M == 1, else written transposed.
        Call t = c;
        t.M = c.N;
        t.N = c.M;
        t.tA = 1 - c.tB;
        t.tB = 1 - c.tA;
        t.A = c.B;
        t.B = c.A;
        t.Aarr = c.Barr;
        t.Barr = c.Aarr;
        t.lda = c.ldb;
        t.ldb = c.lda;
        t.sA = c.sB;
        t.sB = c.sA;
        t.ldc = c.M == 1 ? 1 : c.ldc;
        return launch_gemv(t, s, c.M > 1);
    }

    // Split-K: the tile kernels write per-slice partial tiles into the
    // workspace and a second kernel sums them in slice order.
    const long long part_bytes = 4LL * c.M * c.N * c.batch; // one slice of every item
    int splits = 1, kslice = c.K;
    if (sk.splits == 0 && sk.ws != nullptr) {
        int v = variant;
        long long S = no_split(v) ? 1 : splits_for(v, c.M, c.N, c.K, c.batch, cus, &kslice);
        if (auto_variant && is_stream(v)) {
            // A grid too small even for the streaming kernel's CUs: split the
            // 64 x 64 tile across workgroups instead.
            const int alt = c.K >= 768 ? SGEMM_VARIANT_S64x64_K2 : SGEMM_VARIANT_S64x64;
            const long long S2 = splits_for(alt, c.M, c.N, c.K, c.batch, cus, &kslice);
            if (S2 >= 2) {
                v = alt;
                S = S2;
            }
        }
        const long long fit = (long long)(sk.ws_bytes / (size_t)part_bytes);
        if (S > fit) {
            // Fewer slices, as many as the workspace holds.
            S = fit;
            if (S >= 2) {
                const int bk = kVariants[v].bk;
                const long long ks = ceil_div(ceil_div(c.K, S), bk) * bk;
                kslice = (int)ks;
                S = ceil_div(c.K, ks);
            }
        }
        if (S >= 2) {
            variant = v;
            splits = (int)S;
        } else {
            kslice = c.K;
        }
    } else if (sk.splits >= 2) {
        if (no_split(variant))
            return -19;
        const int bk = kVariants[variant].bk;
        const long long ks = ceil_div(ceil_div(c.K, sk.splits), bk) * bk;
        const long long S = ceil_div(c.K, ks);
        if (S >= 2) {
            if ((size_t)(S * part_bytes) > sk.ws_bytes)
                return -21;
            splits = (int)S;
            kslice = (int)ks;
        }
    }

    if (is_persistent(variant)) {
        if (splits > 1)
            return -19;
        Params p{};
        p.A = c.A;
        p.B = c.B;
        p.C = c.C;
        p.M = c.M;
        p.N = c.N;
        p.K = c.K;
        p.lda = c.lda;
        p.ldb = c.ldb;
        p.ldc = c.ldc;
        p.sA = c.sA;
        p.sB = c.sB;
        p.sC = c.sC;
        p.alpha = c.alpha;
        p.beta = c.beta;
        p.tiles_m = (int)ceil_div(c.M, kVariants[variant].bm);
        p.tiles_n = (int)ceil_div(c.N, kVariants[variant].bn);
        p.group_m = 8;
        p.splits = 1;
        p.kslice = c.K;
        p.slot_tiles = (int)persistent_tiles(variant, c.M, c.N, c.K, c.batch, cus);
        void *args[] = {&p};
        return (int)hipLaunchKernel((const void *)kVariants[variant].fn[c.tA][c.tB],
                                    dim3((unsigned)cus), dim3(768), args, 0, s);
    }

    const VariantInfo &vi = kVariants[variant];
    // One launch holds every tile of an item along grid x, and the runtime
    // counts that axis in work-items (a signed 32-bit range); the tile index
    // inside the kernels is an int as well.
    const long long tiles_item = ceil_div(c.M, vi.bm) * ceil_div(c.N, vi.bn);
    if (tiles_item * vi.threads > INT32_MAX || (long long)splits * tiles_item > INT32_MAX)
        return -22;
    Params p{};
    p.A = c.A;
    p.B = c.B;
    p.C = c.C;
    p.Aarr = c.Aarr;
    p.Barr = c.Barr;
    p.Carr = c.Carr;
    p.M = c.M;
    p.N = c.N;
    p.K = c.K;
    p.lda = c.lda;
    p.ldb = c.ldb;
    p.ldc = c.ldc;
    p.sA = c.sA;
    p.sB = c.sB;
    p.sC = c.sC;
    p.alpha = c.alpha;
    p.beta = c.beta;
    p.tiles_m = (int)ceil_div(c.M, vi.bm);
    p.tiles_n = (int)ceil_div(c.N, vi.bn);
    p.group_m = 8;
    p.splits = splits;
    p.kslice = kslice;
    if (splits > 1) {
        // Partial tiles: C item (batch item, slice) is a dense M x N block of
        // the workspace, written plainly (alpha 1, beta 0).
        p.C = sk.ws;
        p.Carr = nullptr;
        p.ldc = c.N;
        p.sC = (long long)c.M * c.N;
        p.alpha = 1.0f;
        p.beta = 0.0f;
    }
    const long long per_batch = (long long)p.tiles_m * p.tiles_n;
    const long long flat = (long long)c.batch * splits; // workgroup rows: (item, slice)
    // Keep one launch's workgroup count within 2^31 and its batch axis within
    // 65535, in whole items.
    long long max_flat = ((1LL << 31) - 1) / per_batch;
    if (max_flat > 65535)
        max_flat = 65535;
    max_flat -= max_flat % splits; // >= splits: splits * per_batch <= INT32_MAX above
    KernelFn fn = vi.fn[c.tA][c.tB];
    for (long long b0 = 0; b0 < flat; b0 += max_flat) {
        const long long nb = flat - b0 < max_flat ? flat - b0 : max_flat;
        const long long i0 = b0 / splits; // first batch item of this launch
        Params q = p;
        if (arrays) {
            q.Aarr = c.Aarr + i0;
            q.Barr = c.Barr + i0;
            if (splits == 1)
                q.Carr = c.Carr + i0;
        } else {
            q.A = c.A + i0 * c.sA;
            q.B = c.B + i0 * c.sB;
        }
        q.C = splits > 1 ? p.C + b0 * p.sC : (arrays ? nullptr : c.C + i0 * c.sC);
        void *args[] = {&q};
        hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)per_batch, (unsigned)nb),
                                       dim3(vi.threads), args, 0, s);
        if (e != hipSuccess)
            return (int)e;
    }
    if (splits > 1) {
        const long long total = (long long)c.M * c.N * c.batch;
        const long long blocks = ceil_div(total, 256) < 8192 ? ceil_div(total, 256) : 8192;
        const float *W = sk.ws;
        float *C = c.C;
        float *const *Carr = c.Carr;
        int M = c.M, N = c.N, ldc = c.ldc, items = c.batch;
        long long sC = c.sC;
        float alpha = c.alpha, beta = c.beta;
        void *args[] = {&W, &C, &Carr, &M, &N, &ldc, &sC, &items, &splits, &alpha, &beta};
        return (int)hipLaunchKernel((const void *)sgemm_splitk_reduce_kernel, dim3((unsigned)blocks),
                                    dim3(256), args, 0, s);
    }
    return 0;
}

// Column-major arguments checked in their own positions (the same positions
// as the row-major entry points): stored row lengths follow the BLAS
// convention, op(A) M x K with A stored M x K (transA = 0) or K x M, and so on.
int validate_colmajor(int tA, int tB, int M, int N, int K, const float *A, int lda,
                      const float *B, int ldb, const float *C, int ldc, int batch, long long sA,
                      long long sB, long long sC, float alpha, float beta)
{
    if (tA != 0 && tA != 1) return -1;
    if (tB != 0 && tB != 1) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    const int colA = tA ? K : M, colB = tB ? N : K;
    if (lda < (colA > 1 ? colA : 1)) return -8;
    if (ldb < (colB > 1 ? colB : 1)) return -10;
    if (ldc < (M > 1 ? M : 1)) return -13;
    if (batch < 0) return -14;
    if (sA < 0) return -15;
    if (sB < 0) return -16;
    if (sC < 0) return -17;
    const bool work = M > 0 && N > 0 && batch > 0;
    const bool product = work && K > 0 && alpha != 0.0f;
    const bool touch_c = work && (product || beta != 1.0f);
    if (product && A == nullptr) return -7;
    if (product && B == nullptr) return -9;
    if (touch_c && C == nullptr) return -12;
    return 0;
}

} // namespace

extern "C" int sgemm_strided_batched_variant(int transA, int transB, int M, int N, int K,
                                             float alpha, const float *A, int lda,
                                             const float *B, int ldb, float beta, float *C,
                                             int ldc, int batch, long long strideA,
                                             long long strideB, long long strideC, int variant,
                                             sgemm_stream_t stream)
{
    const int st = validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, batch, strideA,
                            strideB, strideC, alpha, beta);
    if (st != 0)
        return st;
    if (variant < SGEMM_VARIANT_AUTO || variant >= SGEMM_VARIANT_COUNT)
        return -18;
    const Call c{transA, transB, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc, batch,
                 strideA, strideB, strideC, nullptr, nullptr, nullptr};
    return launch(c, variant, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int sgemm_strided_batched_ws_variant(int transA, int transB, int M, int N, int K,
                                                float alpha, const float *A, int lda,
                                                const float *B, int ldb, float beta, float *C,
                                                int ldc, int batch, long long strideA,
                                                long long strideB, long long strideC, int variant,
                                                int splits, void *workspace,
                                                size_t workspace_bytes, sgemm_stream_t stream)
{
    const int st = validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, batch, strideA,
                            strideB, strideC, alpha, beta);
    if (st != 0)
        return st;
    if (variant < SGEMM_VARIANT_AUTO || variant >= SGEMM_VARIANT_COUNT)
        return -18;
    if (splits < 0 || splits > 65535)
        return -19;
    if (workspace_bytes > 0 && (workspace == nullptr || ((uintptr_t)workspace & 3u)))
        return -20;
    const Call c{transA, transB, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc, batch,
                 strideA, strideB, strideC, nullptr, nullptr, nullptr};
    const Split sk{workspace_bytes > 0 ? static_cast<float *>(workspace) : nullptr,
                   workspace_bytes, splits};
    return launch(c, variant, reinterpret_cast<hipStream_t>(stream), sk);
}

extern "C" int sgemm_strided_batched_ws(int transA, int transB, int M, int N, int K, float alpha,
                                        const float *A, int lda, const float *B, int ldb,
                                        float beta, float *C, int ldc, int batch,
                                        long long strideA, long long strideB, long long strideC,
                                        void *workspace, size_t workspace_bytes,
                                        sgemm_stream_t stream)
{
    return sgemm_strided_batched_ws_variant(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                                            C, ldc, batch, strideA, strideB, strideC,
                                            SGEMM_VARIANT_AUTO, 0, workspace, workspace_bytes,
                                            stream);
}

extern "C" int sgemm_ws(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                        int lda, const float *B, int ldb, float beta, float *C, int ldc,
                        void *workspace, size_t workspace_bytes, sgemm_stream_t stream)
{
    return sgemm_strided_batched_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                    1, 0, 0, 0, workspace, workspace_bytes, stream);
}

extern "C" size_t sgemm_workspace_size(int transA, int transB, int M, int N, int K, int batch)
{
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1) || M <= 0 || N <= 0 ||
        K <= 0 || batch <= 0)
        return 0;
    int cus = 0;
    if (num_cus_of_current_device(&cus) != 0)
        return 0;
    // The largest split the automatic path makes: it assumes 4-float loads
    // (larger tiles, so no more slices than the 1-float path) and also the
    // 64 x 64 tile that replaces the streaming kernel on tiny grids.
    const int v = sgemm_select_variant(transA, transB, M, N, K, batch, 1, cus);
    int kslice = 0;
    long long S = no_split(v) ? 1 : splits_for(v, M, N, K, batch, cus, &kslice);
    const long long S2 = splits_for(SGEMM_VARIANT_S64x64, M, N, K, batch, cus, &kslice);
    if (is_stream(v) && S2 > S)
        S = S2;
    if (S < 2)
        return 0;
    return (size_t)(S * 4LL * M * N * batch);
}

extern "C" int sgemm_strided_batched(int transA, int transB, int M, int N, int K, float alpha,
                                     const float *A, int lda, const float *B, int ldb,
                                     float beta, float *C, int ldc, int batch, long long strideA,
                                     long long strideB, long long strideC, sgemm_stream_t stream)
{
    return sgemm_strided_batched_variant(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                         ldc, batch, strideA, strideB, strideC,
                                         SGEMM_VARIANT_AUTO, stream);
}

extern "C" int sgemm(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                     int lda, const float *B, int ldb, float beta, float *C, int ldc,
                     sgemm_stream_t stream)
{
    return sgemm_strided_batched(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, 1,
                                 0, 0, 0, stream);
}

extern "C" int sgemm_batched_variant(int transA, int transB, int M, int N, int K, float alpha,
                                     const float *const *A_array, int lda,
                                     const float *const *B_array, int ldb, float beta,
                                     float *const *C_array, int ldc, int batch, int variant,
                                     sgemm_stream_t stream)
{
    // The arrays stand in for the operands in the NULL checks; the item
    // pointers they hold live in device memory and are not inspected here.
    const int st = validate(transA, transB, M, N, K, reinterpret_cast<const float *>(A_array),
                            lda, reinterpret_cast<const float *>(B_array), ldb,
                            reinterpret_cast<const float *>(C_array), ldc, batch, 0, 0, 0, alpha,
                            beta);
    if (st != 0)
        return st;
    if (variant < SGEMM_VARIANT_AUTO || variant >= SGEMM_VARIANT_COUNT)
        return -18;
    // alpha == 0 or K == 0 reads neither A_array nor B_array, which may then be NULL.
    const bool product = K > 0 && alpha != 0.0f;
    const Call c{transA, transB, M, N, K, alpha, beta, nullptr, nullptr, nullptr, lda, ldb, ldc,
                 batch, 0, 0, 0, product ? A_array : nullptr, product ? B_array : nullptr,
                 C_array};
    return launch(c, variant, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int sgemm_batched(int transA, int transB, int M, int N, int K, float alpha,
                             const float *const *A_array, int lda, const float *const *B_array,
                             int ldb, float beta, float *const *C_array, int ldc, int batch,
                             sgemm_stream_t stream)
{
    return sgemm_batched_variant(transA, transB, M, N, K, alpha, A_array, lda, B_array, ldb, beta,
                                 C_array, ldc, batch, SGEMM_VARIANT_AUTO, stream);
}

extern "C" int sgemm_colmajor_strided_batched(int transA, int transB, int M, int N, int K,
                                              float alpha, const float *A, int lda,
                                              const float *B, int ldb, float beta, float *C,
                                              int ldc, int batch, long long strideA,
                                              long long strideB, long long strideC,
                                              sgemm_stream_t stream)
{
    const int st = validate_colmajor(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, batch,
                                     strideA, strideB, strideC, alpha, beta);
    if (st != 0)
        return st;
    // A column-major C (M x N, ld ldc) is, read row-major, C^T (N x M) with the
    // same ld, and C^T = op(B)^T op(A)^T: the row-major product with the
    // operands swapped. A column-major B read row-major is B^T, so op(B)^T is
    // stored exactly as a row-major operand with the same transpose flag, and
    // likewise for A.
    const Call c{transB, transA, N, M, K, alpha, beta, B, A, C, ldb, lda, ldc, batch,
                 strideB, strideA, strideC, nullptr, nullptr, nullptr};
    return launch(c, SGEMM_VARIANT_AUTO, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int sgemm_colmajor(int transA, int transB, int M, int N, int K, float alpha,
                              const float *A, int lda, const float *B, int ldb, float beta,
                              float *C, int ldc, sgemm_stream_t stream)
{
    return sgemm_colmajor_strided_batched(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                          ldc, 1, 0, 0, 0, stream);
}

extern "C" int sgemm_window_ranges(long long left_bytes, int step_bytes, int nsteps,
                                   unsigned int *ranges)
{
    if (step_bytes <= 0 || nsteps < 0 || (nsteps > 0 && ranges == nullptr))
        return -1;
    WindowRange w;
    w.init(left_bytes, step_bytes);
    for (int i = 0; i < nsteps; ++i)
        ranges[i] = w.take();
    return 0;
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: the split-K partial tiles go to a
// fixed device-resident array instead of a caller workspace. Each GPU the
// library runs on holds its own copy of it until the process ends. Host code
// never uses the array's name as an address (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, once per
// device with that device current, and that pointer is what the kernels get.
// Every partial element the reduction reads is written first by the tile
// kernel of the same call, so nothing in the array needs clearing; calls
// that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[SGEMM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float *g_scratch_ptr[kMaxDevices];
int g_scratch_status[kMaxDevices];

// Device address of this device's scratch array (0 on success).
int scratch_of_current_device(float **out)
{
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_status[dev] = (int)r;
        g_scratch_ptr[dev] = r == hipSuccess ? static_cast<float *>(ptr) : nullptr;
    });
    if (g_scratch_status[dev] != 0)
        return g_scratch_status[dev];
    *out = g_scratch_ptr[dev];
    return 0;
}

} // namespace

extern "C" int sgemm_strided_batched_noalloc(int transA, int transB, int M, int N, int K,
                                             float alpha, const float *A, int lda,
                                             const float *B, int ldb, float beta, float *C,
                                             int ldc, int batch, long long strideA,
                                             long long strideB, long long strideC, int splits,
                                             sgemm_stream_t stream)
{
    const int st = validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, batch, strideA,
                            strideB, strideC, alpha, beta);
    if (st != 0)
        return st;
    if (splits < 0 || splits > 65535)
        return -19;
    float *ws = nullptr;
    const int se = scratch_of_current_device(&ws);
    if (se != 0)
        return se;
    const Call c{transA, transB, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc, batch,
                 strideA, strideB, strideC, nullptr, nullptr, nullptr};
    const Split sk{ws, SGEMM_NOALLOC_SCRATCH_BYTES, splits};
    // A forced split whose partial tiles would not fit the array is refused
    // before anything is launched (-21 from the launch path, reported as
    // -23); the automatic choice takes no more slices than fit.
    const int r = launch(c, SGEMM_VARIANT_AUTO, reinterpret_cast<hipStream_t>(stream), sk);
    return r == -21 ? -23 : r;
}

extern "C" const char *sgemm_status_string(int status)
{
    switch (status) {
    case 0: return "success";
    case -1: return "invalid argument 1 (transA must be 0 or 1)";
    case -2: return "invalid argument 2 (transB must be 0 or 1)";
    case -3: return "invalid argument 3 (M < 0)";
    case -4: return "invalid argument 4 (N < 0)";
    case -5: return "invalid argument 5 (K < 0)";
    case -7: return "invalid argument 7 (A or A_array is NULL)";
    case -8: return "invalid argument 8 (lda below the stored row length)";
    case -9: return "invalid argument 9 (B or B_array is NULL)";
    case -10: return "invalid argument 10 (ldb below the stored row length)";
    case -12: return "invalid argument 12 (C or C_array is NULL)";
    case -13: return "invalid argument 13 (ldc below the stored row length)";
    case -14: return "invalid argument 14 (batch < 0)";
    case -15: return "invalid argument 15 (strideA < 0)";
    case -16: return "invalid argument 16 (strideB < 0)";
    case -17: return "invalid argument 17 (strideC < 0)";
    case -18: return "invalid variant argument (unknown variant, a 4-float variant for unaligned operands, or a 32-bit-offset variant for a leading dimension of 2^21 or more)";
    case -19: return "invalid split count (negative, over 65535, or a split of the streaming variant)";
    case -20: return "invalid workspace (NULL or not 4-byte aligned while workspace_bytes > 0)";
    case -21: return "workspace too small for the requested split count";
    case -22: return "problem too large: one batch item has more output tiles than one launch holds";
    case -23: return "split too large: its partial tiles exceed the fixed scratch of the no-allocation entry point (SGEMM_NOALLOC_SCRATCH_BYTES)";
    case -24: return "invalid dispatch override: entries is NULL, or a record has a transpose flag other than 0 or 1, a negative size or a variant that may not be named";
    case -25: return "invalid dispatch override count: negative or above SGEMM_MAX_DISPATCH_OVERRIDES";
    default: break;
    }
    if (status < 0)
        return "invalid argument";
    return hipGetErrorString(static_cast<hipError_t>(status));
}
