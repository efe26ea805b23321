// cbs_device.h -- device-side helpers shared by the gfx950 kernels: element
// types, the fused epilogue, MFMA fragment types and the geometry record.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cbs_shape.h"

namespace cbs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Epilogue of "Fusing an Epilogue" (section "The shape of it"): the folded
// batch norm scales and shifts by the output channel's parameters,
// then SiLU(v) = v * sigmoid(v), sigmoid(v) = 1 / (1 + e^-v).  e^-v is taken
// as 2^(-v*log2 e) on the hardware exp2 unit and the quotient through the
// hardware reciprocal (both about 1 ulp in fp32).  For v below about -88,
// e^-v overflows to +inf, the reciprocal gives 0 and the result is -0, the
// correct limit; for large v the result tends to v.
__device__ __forceinline__ float bn_silu(float acc, float scale, float bias) {
    float v = __builtin_fmaf(acc, scale, bias);
    float e = __builtin_amdgcn_exp2f(v * -1.4426950408889634f);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Round to bfloat16, nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Raw buffer access.  A buffer resource carries the tensor's size in bytes;
// a load at an offset past it returns zero and a store there is dropped, so
// masked lanes need no branch (branches around memory operations make the
// compiler wait for every outstanding access instead of just the ones a
// value depends on).  Offsets are 32-bit, so tensors used this way must stay
// below kMaxBufferBytes.
constexpr uint32_t kOOB = 0xFFFFFFF0u;           // past the end of every buffer
constexpr uint64_t kMaxBufferBytes = 0xFFFFFF00ull;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
// As buf_store16 with the non-temporal (streaming) cache policy.  Measured on
// gfx950: where every store instruction writes whole aligned 64-byte
// segments (four consecutive lanes per segment), y streams out during the
// kernel and the layer runs faster; where a segment is split between
// instructions, or a lane writes 8 bytes, it is markedly slower, so callers
// use it only for whole-segment store patterns.
__device__ __forceinline__ void buf_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ float load(const float *p) { return *p; }
    __device__ static __forceinline__ void store(float *p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store(uint16_t *p, float v) { *p = to_bf16(v); }
};

}  // namespace cbs
