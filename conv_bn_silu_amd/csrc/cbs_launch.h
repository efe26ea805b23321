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

// 1x1, stride 1, pad 0 streaming GEMM (bf16, C_in % 8 == 0, C_in <= 256,
// H*W % 8 == 0); x, w and y 16-byte aligned.
bool pointwise_supports(const Shape &s, int dtype);
bool pointwise_pointers_ok(const void *x, const void *w, const void *y);
hipError_t launch_pointwise(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                            const float *bias, void *y, hipStream_t st, int num_cu);

// Window-staged implicit GEMM (bf16; W, OW multiples of 4), weights
// gathered from OIHW; x 16-byte and y 8-byte aligned.
bool window_supports(const Shape &s, int dtype);
bool window_pointers_ok(const void *x, const void *w, const void *y);
hipError_t launch_window(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                         const float *bias, void *y, hipStream_t st, int num_cu);

// Small-K stem: 3x3, stride 2, pad 1, C_in <= 3, C_out <= 16 (bf16; W a
// multiple of 32, OW <= 320); x and y 16-byte aligned.
bool stem_supports(const Shape &s, int dtype);
bool stem_pointers_ok(const void *x, const void *w, const void *y);
hipError_t launch_stem(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                       const float *bias, void *y, hipStream_t st, int num_cu);

// 3x3 stride-2 pad-1 layers with C_in a multiple of 16 up to 64 (bf16; W a
// multiple of 8, OW a multiple of 4 and at most 160); x, w, y 16-byte
// aligned.
bool rows_supports(const Shape &s, int dtype);
bool rows_pointers_ok(const void *x, const void *w, const void *y);
hipError_t launch_rows(const Shape &s, int epi, const void *x, const void *w, const float *scale, const float *bias,
                       void *y, hipStream_t st, int num_cu);

// Window-staged 3x3 implicit GEMM on 32x32x16 MFMA, 13 or 14 accumulator
// tiles per wave (bf16; W, OW multiples of 4, C_in a multiple of 8), weights
// staged from OIHW; x and w 16-byte, y 8-byte aligned.
// window32_efficiency: share (per mille) of a tile's matrix work that lands
// on real output pixels.
bool window32_supports(const Shape &s, int dtype);
bool window32_pointers_ok(const void *x, const void *w, const void *y);
int window32_efficiency(const Shape &s);
hipError_t launch_window32(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                           const float *bias, void *y, hipStream_t st, int num_cu);

// Each lane computes a single output; any geometry, both dtypes.
bool scalar_supports(const Shape &s, int dtype);
hipError_t launch_scalar(const Shape &s, int dtype, int epi, const void *x, const void *w,
                         const float *scale, const float *bias, void *y, hipStream_t st);

// Device scratch of the allocation-free unfused entry point: t1 and t2, half
// each (cbs_noalloc.hip); its address on the current device.
constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;
hipError_t noalloc_scratch_address(void **out);

// Element-wise passes of the unfused sequence: t2 = t1*scale[co] + bias[co],
// then y = SiLU(t2), each rounded to dtype.
hipError_t launch_bn_pass(const Shape &s, int dtype, const void *t1, const float *scale,
                          const float *bias, void *t2, hipStream_t st);
hipError_t launch_silu_pass(const Shape &s, int dtype, const void *t2, void *y, hipStream_t st);

}  // namespace cbs
