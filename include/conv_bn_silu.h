/*
 * conv_bn_silu.h -- C ABI of the MI355X (gfx950) fused convolution + folded
 * batch norm + SiLU operator.
 *
 * The operation (page "Fusing an Epilogue", sections "The problem" and "The
 * shape of it"): a 2-D convolution computed as a GEMM whose output tile, while
 * still in registers, is scaled and shifted per output channel (folded batch
 * norm: v = acc * scale[co] + bias[co]) and passed through SiLU
 * (y = v * sigmoid(v)) before it is stored.  x is read once and y is written
 * once; the intermediate results of the unfused sequence never reach memory.
 *
 *   y[n][co][oh][ow] = SiLU( scale[co] *
 *        sum_{ci,kh,kw} X(n, ci, oh*stride - pad + kh, ow*stride - pad + kw)
 *                       * w[co][ci][kh][kw]  + bias[co] )
 *
 * where X is x with zeros outside [0,H) x [0,W) (cross-correlation, zero
 * padding, dilation 1, one group) and OH = floor((H + 2*pad - KH)/stride) + 1
 * (OW likewise).  Accumulation and the epilogue run in fp32; the result is
 * rounded once to the output type (round to nearest even for bf16).
 *
 * Conventions shared by every entry point below:
 *   - Layouts: x is contiguous NCHW [N][C_in][H][W]; w is contiguous OIHW
 *     [C_out][C_in][KH][KW]; y is contiguous NCHW [N][C_out][OH][OW]; scale
 *     and bias are contiguous fp32 [C_out].  x, w and y share one element type
 *     `dtype` (CBS_DTYPE_F32 or CBS_DTYPE_BF16, bf16 passed as raw 16-bit
 *     patterns).
 *   - Pointers x, w, scale, bias, y are DEVICE pointers owned by the caller;
 *     the library keeps none of them after a call returns.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream).  Work is enqueued
 *     on that stream and the call returns without waiting; completion is
 *     observed through the stream.
 *   - Every argument is validated on the host before any HIP call, so a
 *     rejected call has no effect on the device.
 *   - Nothing throws across this boundary; every function returns a status.
 */
#ifndef CONV_BN_SILU_H
#define CONV_BN_SILU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    CBS_OK = 0,
    CBS_ERR_INVALID_ARG = 1, /* null pointer, bad size, unknown dtype/variant, overlap */
    CBS_ERR_UNSUPPORTED = 2, /* device is not gfx950, a tensor exceeds 2^31-1 elements, a
                                pointer is not aligned to its element size, or a forced
                                variant cannot run this shape or these pointers */
    CBS_ERR_NO_DEVICE = 3,   /* no HIP device is visible */
    CBS_ERR_HIP = 4,         /* a HIP runtime call failed; see conv_bn_silu_last_hip_error */
    CBS_ERR_BAD_HANDLE = 5   /* NULL, destroyed or foreign handle */
};

/* Element types of x, w and y. */
enum { CBS_DTYPE_F32 = 0, CBS_DTYPE_BF16 = 1 };

/* Kernel variants.  AUTO lets the library choose from the shape (the page's
 * section "Three kernels for one operation": one operator, several kernels,
 * the kernel chosen per shape).  The others force one implementation;
 * they exist so that tests and benchmarks can check each variant on every
 * shape it may serve. */
enum {
    CBS_VARIANT_AUTO = 0,
    CBS_VARIANT_GEMM_GATHER = 1, /* implicit GEMM on MFMA, per-slice gather; any shape */
    CBS_VARIANT_GEMM_WINDOW = 2, /* implicit GEMM on MFMA, input window staged once per
                                    channel block and reused by every kernel tap (bf16) */
    CBS_VARIANT_POINTWISE = 3,   /* 1x1, stride 1, pad 0: streams x once, all output
                                    channels per workgroup (bf16) */
    CBS_VARIANT_SMALL_K = 4,     /* small reduction: the 3x3 stride-2 pad-1 RGB stem
                                    (C_in <= 3, C_out <= 16, W a multiple of 32,
                                    OW <= 320), K = 27 in one MFMA step (bf16) */
    CBS_VARIANT_SCALAR = 5,      /* each lane computes a single output, no tiling; small shapes */
    CBS_VARIANT_GEMM_WINDOW32 = 6, /* as GEMM_WINDOW on 32x32x16 MFMA with larger tiles
                                      per wave: channel-heavy layers (bf16) */
    CBS_VARIANT_ROWS = 7,        /* 3x3 stride-2 pad-1 layers with C_in a multiple of 16
                                    up to 64 (OW <= 160): per-row tap arrays in LDS,
                                    transposed fragment reads (bf16) */
    CBS_VARIANT_COUNT_ = 8
};

typedef struct conv_bn_silu_handle *conv_bn_silu_t;

/* Create a handle bound to the current HIP device.  Queries the device once
 * (graphics IP version, compute-unit count) for dispatch and allocates no
 * device memory.  The handle is read-only from then on, so one handle may
 * serve concurrent calls from any number of threads and streams.
 * Returns CBS_ERR_NO_DEVICE without a visible device, CBS_ERR_UNSUPPORTED if
 * the device is not gfx950, CBS_ERR_INVALID_ARG if out_handle is NULL.
 * On failure *out_handle is set to NULL. */
int conv_bn_silu_create(conv_bn_silu_t *out_handle);

/* Destroy a handle.  Work already enqueued is unaffected (the kernels hold
 * nothing of the handle).  NULL is accepted. */
int conv_bn_silu_destroy(conv_bn_silu_t handle);

/* Enqueue the fused operator on `stream` (see the conventions above).
 * N = 0 is valid and enqueues nothing (the pointers are then not looked at);
 * every other size must be >= 1, stride >= 1, pad >= 0, and the output must be non-empty.
 * y must not overlap x, w, scale or bias (the convolution reads neighbours,
 * so in-place use is not possible): CBS_ERR_INVALID_ARG.  x, w and y must be
 * aligned to their element size, scale and bias to 4 bytes, else
 * CBS_ERR_UNSUPPORTED (16-byte alignment lets the vectorised kernels serve
 * the call; less makes AUTO pick a kernel without vector accesses).
 * The call allocates nothing and takes no workspace: the kernels read the
 * weights in their OIHW layout directly.  It only enqueues kernels, so it is
 * reentrant: calls with one handle on different streams may run
 * concurrently. */
int conv_bn_silu_run(conv_bn_silu_t handle,
                     const void *x, const void *w, const float *scale, const float *bias,
                     void *y,
                     int N, int C_in, int H, int W, int C_out, int KH, int KW,
                     int stride, int pad, int dtype, void *stream);

/* As conv_bn_silu_run, with the kernel variant forced (CBS_VARIANT_*).  A
 * variant that cannot serve the shape, dtype or pointer alignment returns
 * CBS_ERR_UNSUPPORTED. */
int conv_bn_silu_run_variant(conv_bn_silu_t handle, int variant,
                             const void *x, const void *w, const float *scale, const float *bias,
                             void *y,
                             int N, int C_in, int H, int W, int C_out, int KH, int KW,
                             int stride, int pad, int dtype, void *stream);

/* The unfused sequence the fused operator replaces (page "Fusing an
 * Epilogue", section "The problem": conv writes t1, batch norm reads t1 and
 * writes t2, SiLU reads t2 and writes y), as three kernels on `stream`, for
 * measuring the fused kernel against it.  t1 and t2 are caller-owned device
 * buffers of N*C_out*OH*OW elements of `dtype` (intermediates are rounded to
 * dtype, as three separate library calls would store them).  The convolution
 * kernel is the one AUTO dispatch picks for the fused call, run without its
 * epilogue.  Same validation as conv_bn_silu_run; t1 and t2 must not overlap
 * each other or any other buffer (CBS_ERR_INVALID_ARG) and must be aligned
 * like y (CBS_ERR_UNSUPPORTED).  Allocates nothing. */
int conv_bn_silu_run_unfused(conv_bn_silu_t handle,
                             const void *x, const void *w, const float *scale, const float *bias,
                             void *t1, void *t2, void *y,
                             int N, int C_in, int H, int W, int C_out, int KH, int KW,
                             int stride, int pad, int dtype, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * unfused sequence of conv_bn_silu_run_unfused with t1 and t2 held in a
 * static device array of the library -- 64 MiB per GPU, allocated when the
 * library is loaded onto that GPU and kept until the process ends -- so the
 * caller passes only the inputs and y.  Each intermediate (N*C_out*OH*OW
 * elements of `dtype`) may take at most 32 MiB; larger calls return
 * CBS_ERR_UNSUPPORTED before touching the device.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).  Every call on a
 * GPU uses that GPU's one array: calls that overlap in time on one GPU
 * (concurrent streams, threads) race on it and must be serialised by the
 * caller.  Every element of t1 and t2 is written before it is read, so no
 * clearing is needed between calls.  Validation and status codes as
 * conv_bn_silu_run; CBS_ERR_HIP if the array's device address could not be
 * obtained when the handle was created. */
int conv_bn_silu_run_unfused_noalloc(conv_bn_silu_t handle,
                                     const void *x, const void *w, const float *scale, const float *bias,
                                     void *y,
                                     int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                     int stride, int pad, int dtype, void *stream);

/* Host-only helpers (no HIP calls, usable without a device). */

/* Output size OH, OW for the given geometry; CBS_ERR_INVALID_ARG if a size
 * is < 1, stride < 1, pad < 0 or the window does not fit. */
int conv_bn_silu_output_hw(int H, int W, int KH, int KW, int stride, int pad,
                           int *OH, int *OW);

/* The argument checks conv_bn_silu_run performs before touching the device,
 * on their own.  Pointers are only compared and aligned-checked, never read. */
int conv_bn_silu_validate(const void *x, const void *w, const float *scale, const float *bias,
                          const void *y,
                          int N, int C_in, int H, int W, int C_out, int KH, int KW,
                          int stride, int pad, int dtype);

/* The variant AUTO dispatch would choose for this shape on a device with
 * `num_cu` compute units (pass 256 for MI355X).  Returns a CBS_VARIANT_*
 * value, or -1 for an invalid shape. */
int conv_bn_silu_select_variant(int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                int stride, int pad, int dtype, int num_cu);

/* Whether `variant` can run this shape and dtype (1) or not (0). */
int conv_bn_silu_variant_supports(int variant, int N, int C_in, int H, int W, int C_out,
                                  int KH, int KW, int stride, int pad, int dtype);

/* Static, NUL-terminated names; "unknown" for out-of-range values. */
const char *conv_bn_silu_status_string(int status);
const char *conv_bn_silu_variant_name(int variant);

/* The hipError_t of the last failed HIP call the calling thread made through
 * the library (0 if none; kept per thread, not in the handle, so that handles
 * stay read-only).  0 for an invalid handle. */
int conv_bn_silu_last_hip_error(conv_bn_silu_t handle);

/* Fold inference-time batch-norm statistics into the per-channel scale and
 * bias the operator takes (host memory, C_out entries each):
 *   scale[c] = gamma[c] / sqrt(var[c] + eps)
 *   bias[c]  = beta[c] + (conv_bias[c] - mean[c]) * scale[c]
 * conv_bias may be NULL (no convolution bias).  Computed in double, stored
 * as float.  CBS_ERR_INVALID_ARG for NULL arrays, C_out < 1, eps < 0 or a
 * var[c] + eps that is not > 0. */
int conv_bn_silu_fold_bn(const float *gamma, const float *beta, const float *mean,
                         const float *var, float eps, const float *conv_bias, int C_out,
                         float *scale, float *bias);

#ifdef __cplusplus
}
#endif

#endif /* CONV_BN_SILU_H */
