// Test-only probes of the gfx950 FP32 MFMA that the SGEMM kernels rely on.
//
// probe_mfma_layout: one wave runs a single v_mfma_f32_32x32x2_f32 with a zero
// accumulator on the operands the caller gives per lane and writes back every
// lane's 16 accumulator registers, so a test can check the operand and
// accumulator lane layouts against a plain 32x2 by 2x32 product.
//
// probe_mfma_tflops: a grid of workgroups that issue long runs of independent
// MFMAs (no memory traffic) and the elapsed time between two events, as the
// FP32-MFMA rate this device sustains.
//
// probe_mfma_shape_tflops: the same for either FP32 MFMA shape (32x32x2 or
// 16x16x4) with four independent accumulators per wave or a single dependent
// chain, so the rate of each shape and the latency a chain exposes can be
// compared.
#include <hip/hip_runtime.h>

#include <type_traits>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ void __launch_bounds__(64) layout_kernel(const float *a, const float *b, float *d)
{
    const int lane = threadIdx.x;
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[lane], b[lane], acc, 0, 0, 0);
    for (int v = 0; v < 16; ++v)
        d[lane * 16 + v] = acc[v];
}

// Four independent accumulators per wave, `iters` rounds of four MFMAs each.
// The result is written (and depends on every MFMA) so nothing is elided.
__global__ void __launch_bounds__(256) rate_kernel(int iters, float seed, float *out)
{
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    const float x = seed + threadIdx.x * 1e-7f, y = seed - threadIdx.x * 1e-7f;
    for (int i = 0; i < iters; ++i) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(y, x, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, x, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x2f32(y, y, acc3, 0, 0, 0);
    }
    float s = 0.0f;
    for (int v = 0; v < 16; ++v)
        s += acc0[v] + acc1[v] + acc2[v] + acc3[v];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// SHAPE 32: v_mfma_f32_32x32x2_f32 (4096 flop); 16: v_mfma_f32_16x16x4_f32
// (2048 flop). CHAINS independent accumulators, `iters` rounds of four MFMAs
// spread over them (CHAINS = 1: every MFMA waits for the previous one).
template <int SHAPE, int CHAINS>
__global__ void __launch_bounds__(256) shape_kernel(int iters, float seed, float *out)
{
    using Acc = typename std::conditional<SHAPE == 32, f32x16, f32x4>::type;
    constexpr int NV = SHAPE == 32 ? 16 : 4;
    Acc acc[CHAINS];
    for (int c = 0; c < CHAINS; ++c)
        acc[c] = Acc{};
    const float x = seed + threadIdx.x * 1e-7f, y = seed - threadIdx.x * 1e-7f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Acc &a = acc[j % CHAINS];
            if constexpr (SHAPE == 32)
                a = __builtin_amdgcn_mfma_f32_32x32x2f32(j & 1 ? x : y, j & 2 ? y : x, a, 0, 0, 0);
            else
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(j & 1 ? x : y, j & 2 ? y : x, a, 0, 0, 0);
        }
    }
    float s = 0.0f;
    for (int c = 0; c < CHAINS; ++c)
        for (int v = 0; v < NV; ++v)
            s += acc[c][v];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

} // namespace

// a, b: 64 floats each (DEVICE); d: 64 * 16 floats (DEVICE). Synchronous.
extern "C" int probe_mfma_layout(const float *a, const float *b, float *d)
{
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(64), 0, 0, a, b, d);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    return (int)e;
}

// Times 10 launches of `blocks` workgroups of 4 waves, each wave 4 * iters
// MFMAs of 4096 flop, after 100 untimed ones; out: blocks * 256 floats
// (DEVICE). Returns TFLOP/s through *tflops.
extern "C" int probe_mfma_tflops(int blocks, int iters, float *out, double *tflops)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float ms = 0.0f;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess)
        e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        // untimed runs first (tens of ms): the clock ramps up under load
        for (int i = 0; i < 100; ++i)
            hipLaunchKernelGGL(rate_kernel, dim3(blocks), dim3(256), 0, 0, iters, 1.0f, out);
        e = hipEventRecord(e0, 0);
    }
    if (e == hipSuccess) {
        for (int i = 0; i < 10; ++i)
            hipLaunchKernelGGL(rate_kernel, dim3(blocks), dim3(256), 0, 0, iters, 1.0f, out);
        e = hipEventRecord(e1, 0);
    }
    if (e == hipSuccess)
        e = hipGetLastError();
    if (e == hipSuccess)
        e = hipEventSynchronize(e1);
    if (e == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    if (e0 != nullptr)
        (void)hipEventDestroy(e0);
    if (e1 != nullptr)
        (void)hipEventDestroy(e1);
    if (e != hipSuccess)
        return (int)e;
    const double flop = 10.0 * blocks * 4 * 4 * (double)iters * 4096.0;
    *tflops = flop / (ms * 1e-3) / 1e12;
    return 0;
}

// shape: 32 or 16; chains: 1 or 4. Times 10 launches of `blocks` workgroups of
// 4 waves, each wave 4 * iters MFMAs, after 100 untimed ones; out: blocks *
// 256 floats (DEVICE). Returns TFLOP/s through *tflops; -1 for another shape
// or chain count.
extern "C" int probe_mfma_shape_tflops(int shape, int chains, int blocks, int iters, float *out,
                                       double *tflops)
{
    void (*k)(int, float, float *) = nullptr;
    if (shape == 32 && chains == 4) k = shape_kernel<32, 4>;
    if (shape == 32 && chains == 1) k = shape_kernel<32, 1>;
    if (shape == 16 && chains == 4) k = shape_kernel<16, 4>;
    if (shape == 16 && chains == 1) k = shape_kernel<16, 1>;
    if (k == nullptr)
        return -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float ms = 0.0f;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess)
        e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        for (int i = 0; i < 100; ++i)
            hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, iters, 1.0f, out);
        e = hipEventRecord(e0, 0);
    }
    if (e == hipSuccess) {
        for (int i = 0; i < 10; ++i)
            hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, iters, 1.0f, out);
        e = hipEventRecord(e1, 0);
    }
    if (e == hipSuccess)
        e = hipGetLastError();
    if (e == hipSuccess)
        e = hipEventSynchronize(e1);
    if (e == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    if (e0 != nullptr)
        (void)hipEventDestroy(e0);
    if (e1 != nullptr)
        (void)hipEventDestroy(e1);
    if (e != hipSuccess)
        return (int)e;
    const double flop_per = shape == 32 ? 4096.0 : 2048.0;
    const double flop = 10.0 * blocks * 4 * 4 * (double)iters * flop_per;
    *tflops = flop / (ms * 1e-3) / 1e12;
    return 0;
}
