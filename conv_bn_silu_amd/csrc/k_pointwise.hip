// k_pointwise.hip -- the 1x1 (stride 1, no padding) layer as a streaming GEMM.
//
// For a 1x1 convolution the implicit GEMM has no window: row m of the pixel
// operand is x[n][:][p] with m = n*H*W + p, so "read x once, write y once"
// (page "Fusing an Epilogue", section "The problem") means streaming x and y
// through the chip exactly once.  This kernel is built for that:
//
//  * Persistent, statically balanced workgroups.  Workgroup b owns the pixel
//    range [b*P, (b+1)*P) (P a multiple of 8, about M / #workgroups), so
//    every compute unit moves the same number of bytes and there is no tail
//    of half-empty tile waves.  It walks its range in chunks of CP pixels.
//  * Every output channel of a pixel is produced by the same workgroup (up to
//    64*NCB channels per workgroup), so x is fetched from HBM once.
//  * The weights of the workgroup's channels stay in VGPRs for the whole
//    kernel (they are the B operand of every MFMA, 16 bytes per lane each).
//  * x chunks are copied into LDS in their NCHW order ([channel][pixel], 16
//    bytes per lane), and the MFMA A fragments -- eight consecutive channels
//    of one pixel per lane -- are produced by ds_read_b64_tr_b16, which
//    transposes 4x16 blocks of 16-bit values across each 16-lane group.  Rows
//    are padded so that the four rows a group reads fall in distinct banks.
//  * Two chunks of x are in flight in registers while a third is computed.
//  * The epilogue (folded BN, SiLU, bf16 rounding) runs on the accumulators
//    and each lane stores four consecutive pixels of one channel (8 bytes).
#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

constexpr int kThreads = 256;  // 4 waves; wave w owns output channels [16*NCB*w, 16*NCB*(w+1))

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t *lds_elem) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(lds_elem));
    return __builtin_bit_cast(u32x2, v);
}

// NCB: 16-channel blocks per wave; KS: 32-channel slices of C_in (C_in <= 32*KS);
// CP: pixels per chunk; EPI: fused epilogue or the bare convolution.
template <int NCB, int KS, int CP, int EPI>
__global__ __launch_bounds__(kThreads, 1) void pointwise_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int px_per_wg, int co_tiles) {
    constexpr int ROW = CP + 16;                       // LDS elements per channel row
    constexpr int KP = KS * 32;                        // channels held in LDS (zero beyond C_in)
    constexpr int TASKS = (KP * (CP / 8) + kThreads - 1) / kThreads;  // 16-byte copies per thread per chunk
    constexpr int MB = CP / 16;                        // 16-pixel blocks per chunk
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][KP * ROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wg = (int)blockIdx.x / co_tiles, ct = (int)blockIdx.x % co_tiles;
    const int co_wave = ct * (64 * NCB) + wave * (16 * NCB);
    const int m_begin = wg * px_per_wg;
    const int m_end = min(m_begin + px_per_wg, s.M);
    if (m_begin >= m_end) return;  // uniform across the workgroup

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.HW * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.HW * 2u);

    // Weights (B operand): lane holds channel co = co_wave + 16j + (lane&15),
    // k = 32*ks + 8*(lane>>4) .. +7.
    u32x4 wf[NCB][KS];
    float sc[NCB], bi[NCB];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
        const int co = co_wave + 16 * j + (lane & 15);
        sc[j] = co < s.C_out ? scale[co] : 0.f;
        bi[j] = co < s.C_out ? bias[co] : 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = 32 * ks + 8 * (lane >> 4);
            wf[j][ks] = (co < s.C_out && k < s.C_in) ? *(const u32x4 *)(w + co * s.C_in + k)
                                                      : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Channels >= C_in must read as zero: clear both buffers once.
    for (int i = tid; i < 2 * KP * ROW / 8; i += kThreads) ((u32x4 *)&xs[0][0])[i] = u32x4{0u, 0u, 0u, 0u};

    // Copy task t: channel ci = t / (CP/8), 8-pixel piece t % (CP/8).  A piece
    // outside the workgroup's range, or a chunk past the last, gets an
    // out-of-range offset: the load returns zeros and costs no memory traffic.
    const int n_chunks = (m_end - m_begin + CP - 1) / CP;
    auto load_chunk = [&](int c, u32x4 (&r)[TASKS]) {
#pragma unroll
        for (int q = 0; q < TASKS; ++q) {
            const int t = tid + q * kThreads;
            const int ci = t / (CP / 8), piece = t % (CP / 8);
            const int m = m_begin + c * CP + 8 * piece;
            const int n = m / s.HW, p = m - (m / s.HW) * s.HW;
            const bool ok = ci < s.C_in && m < m_end;
            r[q] = buf_load16(xr, ok ? (uint32_t)((n * s.C_in + ci) * s.HW + p) * 2u : kOOB);
        }
    };
    auto store_chunk = [&](int buf, const u32x4 (&r)[TASKS]) {
#pragma unroll
        for (int q = 0; q < TASKS; ++q) {
            const int t = tid + q * kThreads;
            const int ci = t / (CP / 8), piece = t % (CP / 8);
            if (TASKS * kThreads == KP * (CP / 8) || ci < KP)
                *(u32x4 *)&xs[buf][ci * ROW + 8 * piece] = r[q];
        }
    };

    // Transposed-read geometry: lane (g = lane>>4, j = lane&15) reads channel
    // row 8g + (j>>2) (+4 for the upper half) at pixel column 4*(j&3) of a
    // 16-pixel block; it receives channels 8g..8g+7 of pixel j.
    const int tr_row = 8 * (lane >> 4) + ((lane & 15) >> 2);
    const int tr_col = 4 * (lane & 3);

    auto compute_store = [&](int c, int buf) {
        f32x4 acc[MB][NCB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NCB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const uint16_t *base = &xs[buf][(32 * ks + tr_row) * ROW + 16 * i + tr_col];
                const u32x2 lo = ds_read_tr(base);
                const u32x2 hi = ds_read_tr(base + 4 * ROW);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                for (int j = 0; j < NCB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(bf16x8, wf[j][ks]), acc[i][j], 0, 0, 0);
            }
        }
        // Epilogue: lane holds channel co of each block and pixels 4g..4g+3;
        // out-of-range pixels or channels store to an out-of-range offset.
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int m = m_begin + c * CP + 16 * i + 4 * (lane >> 4);
            const int n = m / s.HW, p = m - (m / s.HW) * s.HW;
#pragma unroll
            for (int j = 0; j < NCB; ++j) {
                const int co = co_wave + 16 * j + (lane & 15);
                const bool ok = m < m_end && co < s.C_out;
                const f32x4 v = acc[i][j];
                u32x2 o;
                if (EPI == kFused) {
                    o.x = pack_bf16x2(bn_silu(v[0], sc[j], bi[j]), bn_silu(v[1], sc[j], bi[j]));
                    o.y = pack_bf16x2(bn_silu(v[2], sc[j], bi[j]), bn_silu(v[3], sc[j], bi[j]));
                } else {
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                }
                buf_store8(yr, ok ? (uint32_t)((n * s.C_out + co) * s.HW + p) * 2u : kOOB, o);
            }
        }
    };

    // Pipeline: chunk c is copied to LDS from registers, chunk c+2 is
    // requested into the same registers, then chunk c is multiplied and
    // stored.  Two chunks of loads are always in flight.
    u32x4 r0[TASKS], r1[TASKS];
    load_chunk(0, r0);
    load_chunk(1, r1);
    __syncthreads();  // LDS clear done
    for (int c = 0; c < n_chunks; c += 2) {
        store_chunk(0, r0);
        load_chunk(c + 2, r0);
        __syncthreads();
        compute_store(c, 0);
        if (c + 1 >= n_chunks) break;
        store_chunk(1, r1);
        load_chunk(c + 3, r1);
        __syncthreads();
        compute_store(c + 1, 1);
    }
}

template <int NCB, int KS, int CP, int EPI>
hipError_t launch_pw(const Shape &s, const void *x, const void *w, const float *scale, const float *bias,
                     void *y, hipStream_t st, int num_cu) {
    const int co_tiles = (s.C_out + 64 * NCB - 1) / (64 * NCB);
    int n_wg = num_cu;  // one workgroup per compute unit per channel tile
    int px_per_wg = (s.M + n_wg - 1) / n_wg;
    px_per_wg = (px_per_wg + 7) / 8 * 8;
    n_wg = (s.M + px_per_wg - 1) / px_per_wg;
    hipLaunchKernelGGL((pointwise_bf16<NCB, KS, CP, EPI>), dim3(n_wg * co_tiles), dim3(kThreads), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, px_per_wg,
                       co_tiles);
    return hipGetLastError();
}

}  // namespace

bool pointwise_supports(const Shape &s, int dtype) {
    return dtype == kDtypeBf16 && s.KH == 1 && s.KW == 1 && s.stride == 1 && s.pad == 0 &&
           s.C_in % 8 == 0 && s.C_in <= 256 && s.HW % 8 == 0 &&
           (uint64_t)s.N * s.C_in * s.HW * 2 <= kMaxBufferBytes &&
           (uint64_t)s.N * s.C_out * s.HW * 2 <= kMaxBufferBytes;
}

bool pointwise_pointers_ok(const void *x, const void *w, const void *y) {
    return (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) == 0;
}

hipError_t launch_pointwise(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                            const float *bias, void *y, hipStream_t st, int num_cu) {
    const int ks = (s.C_in + 31) / 32;
    const int ncb = s.C_out <= 64 ? 1 : (s.C_out <= 128 ? 2 : 4);
#define CBS_PW(NCB_, KS_)                                                                       \
    if (ncb == NCB_ && ks <= KS_)                                                               \
        return epi == kFused ? launch_pw<NCB_, KS_, 64, kFused>(s, x, w, scale, bias, y, st, num_cu) \
                             : launch_pw<NCB_, KS_, 64, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
    CBS_PW(1, 2) CBS_PW(1, 4) CBS_PW(1, 8)
    CBS_PW(2, 2) CBS_PW(2, 4) CBS_PW(2, 8)
    CBS_PW(4, 2) CBS_PW(4, 4) CBS_PW(4, 8)
#undef CBS_PW
    return hipErrorInvalidValue;
}

}  // namespace cbs
