/*
 * conv_bn_silu_bench.h -- measurement support exported by the same library
 * as conv_bn_silu.h: the ceilings the benchmark reports beside the published
 * MI355X peaks, so that a layer's roofline fraction can be read against what
 * the chip sustains in the same run.  Not part of the operator.
 *
 * All pointers are device pointers owned by the caller; `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).  Return values: 0 on
 * success, 1 for an invalid argument, 3 without a device, 4 when a HIP call
 * fails.
 */
#ifndef CONV_BN_SILU_BENCH_H
#define CONV_BN_SILU_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compute-unit count, peak shader clock (kHz) and memory clock (kHz) of the
 * current device, as the HIP runtime reports them. */
int conv_bn_silu_bench_device_info(int *num_cu, int *clock_khz, int *mem_clock_khz);

/* The matrix-core ceiling: n_wg workgroups of 4 waves, each wave issuing
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on register
 * operands (no memory access in the loop).  `sink` receives one float per
 * thread (n_wg * 256 floats) so that the work is not optimised away.
 * conv_bn_silu_bench_mfma_flops gives the launch's flop count (2*32*32*16
 * per instruction), or -1 for invalid sizes. */
int conv_bn_silu_bench_mfma(int n_wg, int iters, float *sink, void *stream);
int64_t conv_bn_silu_bench_mfma_flops(int n_wg, int iters);

/* The streaming ceiling: copy `bytes` (a multiple of 16, non-zero; src and
 * dst 16-byte aligned, not overlapping) with one 16-byte load and store per
 * lane, one workgroup of 256 lanes per 4 KiB. */
int conv_bn_silu_bench_copy(const void *src, void *dst, uint64_t bytes, void *stream);

/* LDS bank-conflict probe: one wave (one workgroup of 64 lanes) repeats one
 * LDS operation 256 times, lane l at byte address addr[l] of a 64 KiB LDS
 * array (masked to it and aligned down to the operation's size).  op: 0
 * ds_read_b128, 1 ds_read_b64, 2 ds_read_b64_tr_b16, 3 ds_write_b64,
 * 4 ds_write_b128.  addr: 64 device uint32; out: 64 device uint32 that
 * receive a checksum.  Read SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS around the
 * dispatch (the kernel first writes its 64 KiB with 64 conflict-free
 * 16-byte stores per lane). */
int conv_bn_silu_bench_lds(int op, const uint32_t *addr, uint32_t *out, void *stream);

/* Instruction-issue probe: n_wg workgroups of 4 waves, each lane running
 * `iters` iterations of register-only work with 8 independent chains:
 * kind 0 v_fma_f32, 1 v_exp_f32, 2 v_add_f32 + v_rcp_f32, 3 the BN + SiLU
 * epilogue (2 fma, exp, add, rcp, mul); kind 10 + NV/8 for NV = 0, 8, 16,
 * 32, 64: 8 v_mfma_f32_32x32x16_bf16 on independent accumulators per
 * iteration with NV independent v_fma_f32 among them.  sink receives one
 * float per thread (n_wg * 256). */
int conv_bn_silu_bench_isa(int kind, int n_wg, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV_BN_SILU_BENCH_H */
