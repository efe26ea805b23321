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
//    hundreds of short workgroups in flight, the stores with the
//    non-temporal policy (about 6.3 TB/s of read + write traffic at 1 GiB
//    each way, 6.2 with ordinary stores; about 5.2 for persistent workgroups
//    walking contiguous chunks and 4.3 for a grid-stride loop).
//  * lds_probe: one wave repeating one LDS operation (16- or 8-byte read or
//    write, or the transposed 8-byte read) at per-lane addresses given by the
//    caller, so that the LDS bank-conflict counter can be read per address
//    pattern.
//  * isa_probe: register-only loops that time instruction issue: fused
//    multiply-adds, the hardware exp2 and reciprocal, the BN + SiLU epilogue
//    sequence, and v_mfma_f32_32x32x16_bf16 with 0..64 independent FMAs
//    issued between each 8 of them (how much vector work one wave hides
//    under its own matrix instructions).
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

constexpr int kLdsIters = 256;

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define CBS_LDS(T, p) (*(volatile __attribute__((address_space(3))) T *)(p))

// OP: 0 ds_read_b128, 1 ds_read_b64, 2 ds_read_b64_tr_b16, 3 ds_write_b64,
// 4 ds_write_b128.  64 KiB of LDS; addresses masked into it and aligned.
template <int OP>
__global__ __launch_bounds__(64) void lds_probe(const uint32_t *__restrict__ addr, uint32_t *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
    const int lane = threadIdx.x;
    for (int i = lane; i < 65536 / 16; i += 64) *(u32x4 *)(lds + 16 * i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    uint32_t a = addr[lane] & ((OP == 0 || OP == 4) ? 0xFFF0u : 0xFFF8u);
    asm volatile("" : "+v"(a));
    u32x4 acc{0u, 0u, 0u, 0u};
    for (int it = 0; it < kLdsIters; ++it) {
        if constexpr (OP == 0) {
            acc += CBS_LDS(u32x4, lds + a);
        } else if constexpr (OP == 1) {
            const u32x2 v = CBS_LDS(u32x2, lds + a);
            acc.x += v.x;
            acc.y += v.y;
        } else if constexpr (OP == 2) {
            const s16x4 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(lds + a));
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            acc.x += w.x;
            acc.y += w.y;
        } else if constexpr (OP == 3) {
            CBS_LDS(u32x2, lds + a) = u32x2{acc.x + (uint32_t)it, acc.y};
        } else {
            CBS_LDS(u32x4, lds + a) = acc + u32x4{(uint32_t)it, 0u, 0u, 0u};
        }
        asm volatile("" : "+v"(acc));
    }
    out[lane] = acc.x + acc.y + acc.z + acc.w;
}
#undef CBS_LDS

// KIND 0..3: 8 independent chains per lane of (0) fma, (1) exp2, (2) add +
// reciprocal, (3) the epilogue (fma, fma, exp2, add, reciprocal, multiply);
// KIND 10 + NV/8 (NV in 0, 8, 16, 32, 64): 8 independent MFMAs per
// iteration with NV independent fmas among them.
template <int KIND>
__global__ __launch_bounds__(kCeilThreads) void isa_probe(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.01f * (float)((lane + j) & 63) - 0.3f;
    if constexpr (KIND < 10) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if constexpr (KIND == 0) v[j] = __builtin_fmaf(v[j], 0.999f, 0.001f);
                if constexpr (KIND == 1) v[j] = __builtin_amdgcn_exp2f(-v[j]);
                if constexpr (KIND == 2) v[j] = __builtin_amdgcn_rcpf(v[j] + 1.0f);
                if constexpr (KIND == 3) {
                    const float x = __builtin_fmaf(v[j], 0.9f, 0.01f);
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(v[j], -1.3f, -0.014f));
                    v[j] = x * __builtin_amdgcn_rcpf(1.0f + e);
                }
            }
        }
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += v[j];
        sink[blockIdx.x * kCeilThreads + threadIdx.x] = t;
    } else {
        constexpr int NV = 8 * (KIND - 10);
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(0.001f * (float)(lane + i));
            b[i] = (__bf16)(0.002f * (float)(lane - i));
        }
        f32x16 acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
                for (int k = 0; k < NV / 8; ++k) v[k] = __builtin_fmaf(v[k], 0.999f, 0.001f);
            }
        }
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) t += acc[c][e];
#pragma unroll
        for (int j = 0; j < 8; ++j) t += v[j];
        sink[blockIdx.x * kCeilThreads + threadIdx.x] = t;
    }
}

__global__ __launch_bounds__(kCeilThreads) void copy16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(src[i], &dst[i]);
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

int conv_bn_silu_bench_lds(int op, const uint32_t *addr, uint32_t *out, void *stream) {
    if (!addr || !out || op < 0 || op > 4) return 1;
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    switch (op) {
    case 0: hipLaunchKernelGGL(cbs::lds_probe<0>, dim3(1), dim3(64), 0, st, addr, out); break;
    case 1: hipLaunchKernelGGL(cbs::lds_probe<1>, dim3(1), dim3(64), 0, st, addr, out); break;
    case 2: hipLaunchKernelGGL(cbs::lds_probe<2>, dim3(1), dim3(64), 0, st, addr, out); break;
    case 3: hipLaunchKernelGGL(cbs::lds_probe<3>, dim3(1), dim3(64), 0, st, addr, out); break;
    default: hipLaunchKernelGGL(cbs::lds_probe<4>, dim3(1), dim3(64), 0, st, addr, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int conv_bn_silu_bench_isa(int kind, int n_wg, int iters, float *sink, void *stream) {
    if (!sink || n_wg < 1 || iters < 1) return 1;
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    const dim3 g(n_wg), b(cbs::kCeilThreads);
    switch (kind) {
    case 0: hipLaunchKernelGGL(cbs::isa_probe<0>, g, b, 0, st, iters, sink); break;
    case 1: hipLaunchKernelGGL(cbs::isa_probe<1>, g, b, 0, st, iters, sink); break;
    case 2: hipLaunchKernelGGL(cbs::isa_probe<2>, g, b, 0, st, iters, sink); break;
    case 3: hipLaunchKernelGGL(cbs::isa_probe<3>, g, b, 0, st, iters, sink); break;
    case 10: hipLaunchKernelGGL(cbs::isa_probe<10>, g, b, 0, st, iters, sink); break;
    case 11: hipLaunchKernelGGL(cbs::isa_probe<11>, g, b, 0, st, iters, sink); break;
    case 12: hipLaunchKernelGGL(cbs::isa_probe<12>, g, b, 0, st, iters, sink); break;
    case 14: hipLaunchKernelGGL(cbs::isa_probe<14>, g, b, 0, st, iters, sink); break;
    case 18: hipLaunchKernelGGL(cbs::isa_probe<18>, g, b, 0, st, iters, sink); break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
