// cbs_launch.h -- host-side entry points of the kernel files, used by the C
// ABI layer (cbs_api.cpp).  Each launcher enqueues its kernels on the given
// stream and returns hipGetLastError() of the launch; callers have validated
// every argument and checked `*_supports` first.
#pragma once

#include <hip/hip_runtime.h>

#include "cbs_shape.h"

namespace cbs {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// Implicit GEMM, per-slice gather; any geometry, both dtypes.
bool gemm_gather_supports(const Shape &s, int dtype);
hipError_t launch_gemm_gather(const Shape &s, int dtype, int epi, const void *x, const void *w,
                              const float *scale, const float *bias, void *y, hipStream_t st);

// One output element per lane; any geometry, both dtypes.
bool scalar_supports(const Shape &s, int dtype);
hipError_t launch_scalar(const Shape &s, int dtype, int epi, const void *x, const void *w,
                         const float *scale, const float *bias, void *y, hipStream_t st);

// Element-wise passes of the unfused sequence: t2 = t1*scale[co] + bias[co],
// then y = SiLU(t2), each rounded to dtype.
hipError_t launch_bn_pass(const Shape &s, int dtype, const void *t1, const float *scale,
                          const float *bias, void *t2, hipStream_t st);
hipError_t launch_silu_pass(const Shape &s, int dtype, const void *t2, void *y, hipStream_t st);

}  // namespace cbs
