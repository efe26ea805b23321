// k_scalar.hip -- the scalar variant (each lane computes one output, page
// "Fusing an Epilogue", section "Three kernels for one operation"), and the
// element-wise batch-norm and SiLU passes of the unfused sequence the fused
// operator replaces (same page, section "The problem").
//
// The scalar kernel has no setup: each lane walks the whole reduction for one
// output in the order ci, kh, kw with fp32 fused multiply-adds and applies
// the epilogue to its own result (a 3x3 form with unrolled, branch-free taps
// serves the common filter).  Lanes run along ow, so loads of x and the
// store of y are coalesced along rows.
#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

constexpr int kThreads = 256;

// Grid-stride loop indices.  The stride (grid x 256) is added in 64 bits and
// the loop ends once the sum passes `total`, so an index never wraps past
// 2^31 - 1 for any total up to INT32_MAX.
__device__ __forceinline__ int first_index() { return (int)(blockIdx.x * kThreads + threadIdx.x); }
__device__ __forceinline__ int next_index(int idx, int total) {
    const long long nxt = (long long)idx + (long long)gridDim.x * kThreads;
    return nxt < total ? (int)nxt : total;
}

template <typename T, int EPI>
__global__ __launch_bounds__(kThreads) void conv_scalar(const T *__restrict__ x, const T *__restrict__ w,
                                                        const float *__restrict__ scale,
                                                        const float *__restrict__ bias, T *__restrict__ y,
                                                        Shape s) {
    const int total = s.N * s.C_out * s.OHW;
    for (int idx = first_index(); idx < total; idx = next_index(idx, total)) {
        const int ow = idx % s.OW;
        const int oh = (idx / s.OW) % s.OH;
        const int co = (idx / s.OHW) % s.C_out;
        const int n = idx / (s.OHW * s.C_out);
        const int ih0 = oh * s.stride - s.pad, iw0 = ow * s.stride - s.pad;
        const T *xn = x + (size_t)n * s.C_in * s.HW;
        const T *wc = w + (size_t)co * s.K;
        float acc = 0.f;
        for (int ci = 0; ci < s.C_in; ++ci) {
            for (int kh = 0; kh < s.KH; ++kh) {
                const int ih = ih0 + kh;
                if ((unsigned)ih >= (unsigned)s.H) continue;
                for (int kw = 0; kw < s.KW; ++kw) {
                    const int iw = iw0 + kw;
                    if ((unsigned)iw >= (unsigned)s.W) continue;
                    acc = __builtin_fmaf(Elem<T>::load(xn + ci * s.HW + ih * s.W + iw),
                                         Elem<T>::load(wc + (ci * s.KH + kh) * s.KW + kw), acc);
                }
            }
        }
        Elem<T>::store(y + idx, EPI == kFused ? bn_silu(acc, scale[co], bias[co]) : acc);
    }
}

// The same operation for 3x3 filters with the taps unrolled and the padding
// applied by masking rather than branching (an out-of-image tap loads from a
// clamped in-image address and is multiplied by zero), so that a lane's loads
// are independent of each other and issue back to back; the channel loop is
// unrolled by four for the same reason.  Same summation order as above.
template <typename T, int EPI>
__global__ __launch_bounds__(kThreads) void conv_scalar3x3(const T *__restrict__ x, const T *__restrict__ w,
                                                           const float *__restrict__ scale,
                                                           const float *__restrict__ bias, T *__restrict__ y,
                                                           Shape s) {
    const int total = s.N * s.C_out * s.OHW;
    for (int idx = first_index(); idx < total; idx = next_index(idx, total)) {
        const int ow = idx % s.OW;
        const int oh = (idx / s.OW) % s.OH;
        const int co = (idx / s.OHW) % s.C_out;
        const int n = idx / (s.OHW * s.C_out);
        const int ih0 = oh * s.stride - s.pad, iw0 = ow * s.stride - s.pad;
        int off[9];
        float msk[9];
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int ih = ih0 + kh, iw = iw0 + kw;
                const bool in = (unsigned)ih < (unsigned)s.H && (unsigned)iw < (unsigned)s.W;
                off[kh * 3 + kw] = in ? ih * s.W + iw : 0;
                msk[kh * 3 + kw] = in ? 1.f : 0.f;
            }
        const T *xn = x + (size_t)n * s.C_in * s.HW;
        const T *wc = w + (size_t)co * s.K;
        float acc = 0.f;
#pragma unroll 4
        for (int ci = 0; ci < s.C_in; ++ci) {
            const T *xc = xn + ci * s.HW;
#pragma unroll
            for (int t = 0; t < 9; ++t)
                acc = __builtin_fmaf(Elem<T>::load(xc + off[t]) * msk[t], Elem<T>::load(wc + ci * 9 + t), acc);
        }
        Elem<T>::store(y + idx, EPI == kFused ? bn_silu(acc, scale[co], bias[co]) : acc);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void bn_pass(const T *__restrict__ t1, const float *__restrict__ scale,
                                                    const float *__restrict__ bias, T *__restrict__ t2,
                                                    int total, int C_out, int OHW) {
    for (int idx = first_index(); idx < total; idx = next_index(idx, total)) {
        const int co = (idx / OHW) % C_out;
        Elem<T>::store(t2 + idx, __builtin_fmaf(Elem<T>::load(t1 + idx), scale[co], bias[co]));
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void silu_pass(const T *__restrict__ t2, T *__restrict__ y, int total) {
    for (int idx = first_index(); idx < total; idx = next_index(idx, total)) {
        const float v = Elem<T>::load(t2 + idx);
        // SiLU alone: the epilogue helper with scale 1 and bias 0.
        Elem<T>::store(y + idx, bn_silu(v, 1.f, 0.f));
    }
}

unsigned grid_for(int total) {
    const long blocks = ((long)total + kThreads - 1) / kThreads;
    return (unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

bool scalar_supports(const Shape &, int) { return true; }

hipError_t launch_scalar(const Shape &s, int dtype, int epi, const void *x, const void *w,
                         const float *scale, const float *bias, void *y, hipStream_t st) {
    const dim3 grid(grid_for(s.N * s.C_out * s.OHW)), block(kThreads);
    const bool k3 = s.KH == 3 && s.KW == 3;
    if (dtype == kDtypeBf16) {
        auto xx = (const uint16_t *)x;
        auto ww = (const uint16_t *)w;
        auto yy = (uint16_t *)y;
        if (k3 && epi == kFused) hipLaunchKernelGGL((conv_scalar3x3<uint16_t, kFused>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else if (k3) hipLaunchKernelGGL((conv_scalar3x3<uint16_t, kConvOnly>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else if (epi == kFused) hipLaunchKernelGGL((conv_scalar<uint16_t, kFused>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else hipLaunchKernelGGL((conv_scalar<uint16_t, kConvOnly>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
    } else {
        auto xx = (const float *)x;
        auto ww = (const float *)w;
        auto yy = (float *)y;
        if (k3 && epi == kFused) hipLaunchKernelGGL((conv_scalar3x3<float, kFused>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else if (k3) hipLaunchKernelGGL((conv_scalar3x3<float, kConvOnly>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else if (epi == kFused) hipLaunchKernelGGL((conv_scalar<float, kFused>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else hipLaunchKernelGGL((conv_scalar<float, kConvOnly>), grid, block, 0, st, xx, ww, scale, bias, yy, s);
    }
    return hipGetLastError();
}

hipError_t launch_bn_pass(const Shape &s, int dtype, const void *t1, const float *scale, const float *bias,
                          void *t2, hipStream_t st) {
    const int total = s.N * s.C_out * s.OHW;
    const dim3 grid(grid_for(total)), block(kThreads);
    if (dtype == kDtypeBf16)
        hipLaunchKernelGGL(bn_pass<uint16_t>, grid, block, 0, st, (const uint16_t *)t1, scale, bias,
                           (uint16_t *)t2, total, s.C_out, s.OHW);
    else
        hipLaunchKernelGGL(bn_pass<float>, grid, block, 0, st, (const float *)t1, scale, bias, (float *)t2,
                           total, s.C_out, s.OHW);
    return hipGetLastError();
}

hipError_t launch_silu_pass(const Shape &s, int dtype, const void *t2, void *y, hipStream_t st) {
    const int total = s.N * s.C_out * s.OHW;
    const dim3 grid(grid_for(total)), block(kThreads);
    if (dtype == kDtypeBf16)
        hipLaunchKernelGGL(silu_pass<uint16_t>, grid, block, 0, st, (const uint16_t *)t2, (uint16_t *)y, total);
    else
        hipLaunchKernelGGL(silu_pass<float>, grid, block, 0, st, (const float *)t2, (float *)y, total);
    return hipGetLastError();
}

}  // namespace cbs
