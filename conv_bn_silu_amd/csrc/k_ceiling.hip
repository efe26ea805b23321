// k_ceiling.hip -- measured ceilings for the benchmark (declared in
// include/conv_bn_silu_bench.h): what the matrix cores and HBM of the GPU the
// operator runs on actually sustain, reported beside the published peaks.
//
//  * mfma_loop: v_mfma_f32_32x32x16_bf16 on register operands only -- no
//    memory traffic inside the loop -- with eight independent accumulators
//    per wave, so that the matrix pipe never waits on a result.
//  * copy16: a streaming copy in its fastest measured form on MI355X: one
//    16-byte load and store per lane, one workgroup per 4 KiB, so every wave
//    instruction covers 1 KiB of contiguous memory and the hardware keeps
//    hundreds of short workgroups in flight (about 6.2 TB/s of read + write
//    traffic, against about 5.2 for persistent workgroups walking contiguous
//    chunks and 4.3 for a grid-stride loop).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/conv_bn_silu_bench.h"
#include "cbs_device.h"

namespace cbs {
namespace {

constexpr int kCeilThreads = 256;
constexpr int kChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(kCeilThreads) void mfma_loop(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) t += acc[c][e];
    sink[blockIdx.x * kCeilThreads + threadIdx.x] = t;
}

__global__ __launch_bounds__(kCeilThreads) void copy16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

}  // namespace
}  // namespace cbs

extern "C" {

int conv_bn_silu_bench_device_info(int *num_cu, int *clock_khz, int *mem_clock_khz) {
    if (!num_cu || !clock_khz || !mem_clock_khz) return 1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 3;
    if (hipDeviceGetAttribute(num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess ||
        hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess)
        return 4;
    return 0;
}

int64_t conv_bn_silu_bench_mfma_flops(int n_wg, int iters) {
    if (n_wg < 1 || iters < 1) return -1;
    // 4 waves per workgroup, kChains instructions per iteration, 2*32*32*16
    // flops per instruction
    return (int64_t)n_wg * 4 * iters * cbs::kChains * 2 * 32 * 32 * 16;
}

int conv_bn_silu_bench_mfma(int n_wg, int iters, float *sink, void *stream) {
    if (n_wg < 1 || iters < 1 || !sink) return 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(cbs::mfma_loop, dim3(n_wg), dim3(cbs::kCeilThreads), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int conv_bn_silu_bench_copy(const void *src, void *dst, uint64_t bytes, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 1;
    const uint64_t n_wg = (bytes / 16 + cbs::kCeilThreads - 1) / cbs::kCeilThreads;
    if (n_wg > 0x7FFFFFFFull) return 1;
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + bytes && d < s + bytes) return 1;  // overlap
    (void)hipGetLastError();
    hipLaunchKernelGGL(cbs::copy16, dim3((unsigned)n_wg), dim3(cbs::kCeilThreads), 0, (hipStream_t)stream,
                       (const cbs::u32x4 *)src, (cbs::u32x4 *)dst, (uint64_t)(bytes / 16));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
