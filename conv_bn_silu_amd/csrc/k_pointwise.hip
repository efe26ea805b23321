// k_pointwise.hip -- the 1x1 (stride 1, no padding) layer as a streaming GEMM.
//
// For a 1x1 convolution the implicit GEMM has no window: row m of the pixel
// operand is x[n][:][p] with m = n*H*W + p, so "read x once, write y once"
// (page "Fusing an Epilogue", section "The problem") means streaming x and y
// through the chip exactly once.  This kernel is built for that:
//
//  * Persistent, statically balanced workgroups, one per compute unit, of 8
//    waves (two per SIMD).  Each owns a pixel range of P pixels (P a multiple
//    of 8, about M / #ranges) and a tile of 256 output channels, so every
//    compute unit moves the same number of bytes and there is no tail of
//    half-empty tile waves.  It walks its range in chunks of CP pixels.
//  * XCD-aware placement: each XCD runs a contiguous run of pixel ranges (and
//    every channel tile of them), so cache lines shared by neighbouring
//    ranges, and x re-read by several channel tiles, meet in one L2.
//  * The weights of each wave's 32 channels stay in VGPRs for the whole
//    kernel (they are the B operand of every MFMA, 16 bytes per lane each).
//  * The products run on v_mfma_f32_32x32x16_bf16 (32 pixels x 32 channels x
//    16 k per instruction), the shape that sustains the matrix-core rate with
//    one wave per SIMD.
//  * x chunks are copied into LDS in their NCHW order ([channel][pixel], 16
//    bytes per lane), and the MFMA A fragments -- eight consecutive channels
//    of one pixel per lane -- are produced by ds_read_b64_tr_b16, which
//    transposes 4x16 blocks of 16-bit values across each 16-lane group.  Rows
//    are padded so that the four rows a group reads fall in distinct banks.
//  * Three chunks of x are in flight in registers while one is computed.
//  * The epilogue (folded BN, SiLU, bf16 rounding) runs on the accumulators;
//    each wave stages its 32-channel output tile in LDS and writes y in whole
//    128-byte rows, 16 bytes per lane.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t *lds_elem) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(lds_elem));
    return __builtin_bit_cast(u32x2, v);
}

// Calls f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Pixel position (image n, offset p within the image) of a chunk start, and
// of the pixel `d` further on (d < H*W: at most one image boundary).
struct PixPos {
    int n, p;
};
__device__ __forceinline__ PixPos advance(PixPos a, int d, int hw) {
    PixPos r{a.n, a.p + d};
    if (r.p >= hw) {
        r.p -= hw;
        ++r.n;
    }
    return r;
}
__device__ __forceinline__ PixPos chunk_start(PixPos start0, int offset, int hw) {
    PixPos c = start0;
    while (offset >= hw) {  // uniform; only for images smaller than a chunk
        offset -= hw;
        ++c.n;
    }
    return advance(c, offset, hw);
}

constexpr int kWaves = 8;               // wave w owns output channels [32w, 32w+32) of the tile
constexpr int kThreadsPw = 64 * kWaves;
constexpr int kTileCo = 32 * kWaves;    // output channels per workgroup

// KS: 16-channel slices of C_in (C_in <= 16*KS); CP: pixels per chunk; PD:
// chunks in flight; EPI: fused epilogue or the bare convolution.
template <int KS, int CP, int PD, int EPI>
__global__ __launch_bounds__(kThreadsPw, 1) void pointwise_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int px_per_wg, int co_tiles,
    int n_ranges, int ranges_per_xcd) {
    constexpr int ROW = CP + 16;                       // x chunk: LDS elements per channel row
    constexpr int KP = KS * 16;                        // channels held in LDS (zero beyond C_in)
    constexpr int TASKS = (KP * (CP / 8) + kThreadsPw - 1) / kThreadsPw;  // 16-byte copies per thread
    constexpr int MB = CP / 32;                        // 32-pixel blocks per chunk
    constexpr int OROW = CP + 8;                       // output staging: elements per channel row
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][KP * ROW];
    __shared__ __attribute__((aligned(16))) uint16_t os[kWaves][32 * OROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Block id -> (pixel range, channel tile), XCD-aware.  The XCDs take
    // workgroups round-robin (XCD = id % 8), so XCD x gets a contiguous run
    // of ranges_per_xcd pixel ranges and all channel tiles of each: ranges
    // that share cache lines at their ends, and the tiles that read the same
    // x, meet in one L2.
    int wg, ct;
    {
        const int b = (int)blockIdx.x;
        const int xcd = b & 7, slot = b >> 3;
        ct = slot % co_tiles;
        const int idx = slot / co_tiles;
        if (idx >= ranges_per_xcd) return;  // uniform
        wg = xcd * ranges_per_xcd + idx;
        if (wg >= n_ranges) return;  // uniform
    }
    const int co_lane = ct * kTileCo + wave * 32 + (lane & 31);  // this lane's output channel
    const int m_begin = wg * px_per_wg;
    const int m_end = min(m_begin + px_per_wg, s.M);
    if (m_begin >= m_end) return;  // uniform across the workgroup
    const int hw = s.HW;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * hw * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * hw * 2u);

    u32x4 wf[KS];  // weights, filled after the first x requests
    float sc, bi, sn, bn;

    const PixPos start0{m_begin / hw, m_begin - (m_begin / hw) * hw};
    const int n_chunks = (m_end - m_begin + CP - 1) / CP;

    // Copy task t: channel ci = t / (CP/8), 8-pixel piece t % (CP/8).  A piece
    // outside the workgroup's range, a channel past C_in, or a chunk past the
    // last, gets an out-of-range offset: the load returns zeros and costs no
    // memory traffic.
    auto load_chunk = [&](int c, u32x4 (&r)[TASKS]) {
        const PixPos c0 = chunk_start(start0, c * CP, hw);
        const int mc = m_begin + c * CP;
#pragma unroll
        for (int q = 0; q < TASKS; ++q) {
            const int t = tid + q * kThreadsPw;
            const int ci = t / (CP / 8), piece = t % (CP / 8);
            const PixPos pp = advance(c0, 8 * piece, hw);
            const bool ok = ci < s.C_in && mc + 8 * piece < m_end;
            r[q] = buf_load16(xr, ok ? (uint32_t)((pp.n * s.C_in + ci) * hw + pp.p) * 2u : kOOB);
        }
    };
    auto store_chunk = [&](int buf, const u32x4 (&r)[TASKS]) {
#pragma unroll
        for (int q = 0; q < TASKS; ++q) {
            const int t = tid + q * kThreadsPw;
            const int ci = t / (CP / 8), piece = t % (CP / 8);
            if (TASKS * kThreadsPw == KP * (CP / 8) || ci < KP)
                *(u32x4 *)&xs[buf][ci * ROW + 8 * piece] = r[q];
        }
    };

    // Transposed-read geometry for the 32x32x16 A operand (lane l: pixel
    // l&31, channels 8*(l>>5) .. +7 of the slice): 16-lane group G = l>>4
    // covers pixels 16*(G&1) .. +15 and channel half G>>1; lane j = l&15 of
    // the group reads channel row 8*(G>>1) + (j>>2) (+4 for the upper four)
    // at pixel column 16*(G&1) + 4*(j&3).
    const int grp = lane >> 4, jl = lane & 15;
    const int tr_row = 8 * (grp >> 1) + (jl >> 2);
    const int tr_col = 16 * (grp & 1) + 4 * (jl & 3);
    uint16_t *const ow = os[wave];

    // MFMAs of one chunk into `acc` (MB 32-pixel blocks).  The A fragments
    // of slice ks+PFD are read while the MFMAs of slice ks run.
    auto read_a = [&](int buf, int ks, int i) {
        const uint16_t *base = &xs[buf][(16 * ks + tr_row) * ROW + 32 * i + tr_col];
        const u32x2 lo = ds_read_tr(base);
        const u32x2 hi = ds_read_tr(base + 4 * ROW);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    };
    auto mfma_chunk = [&](int buf, f32x16 (&acc)[MB]) {
        constexpr int PFD = 2;
        bf16x8 afr[PFD + 1][MB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
#pragma unroll
        for (int p = 0; p < PFD && p < KS; ++p)
#pragma unroll
            for (int i = 0; i < MB; ++i) afr[p][i] = read_a(buf, p, i);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + PFD < KS) {
#pragma unroll
                for (int i = 0; i < MB; ++i) afr[(ks + PFD) % (PFD + 1)][i] = read_a(buf, ks + PFD, i);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[ks % (PFD + 1)][i],
                                                                  __builtin_bit_cast(bf16x8, wf[ks]), acc[i], 0, 0, 0);
        }
    };

    // Epilogue of chunk c from `acc`, in two steps so that y is written in
    // whole rows.  (1) Each lane applies BN + SiLU to its accumulators -- its
    // channel, pixels 8q + 4*(lane>>5) .. +3 of each block -- and writes them,
    // as bf16, to the wave's staging tile [32 channels][CP pixels].  (2) The
    // wave reads the tile back 16 bytes per lane and stores channel rows of y.
    const int row = lane & 31;
    auto epi_math = [&](const f32x16 (&acc)[MB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = acc[i][4 * q + r];
                    if (EPI == kFused) {
                        const float vv = __builtin_fmaf(a, sc, bi);
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(a, sn, bn));
                        o[r] = vv * __builtin_amdgcn_rcpf(1.0f + e);
                    } else {
                        o[r] = a;
                    }
                }
                *(u32x2 *)&ow[row * OROW + 32 * i + 8 * q + 4 * (lane >> 5)] =
                    u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
        }
    };
    auto epi_store = [&](int c, bool live) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        const PixPos c0 = chunk_start(start0, (live ? c : 0) * CP, hw);
        const int mc = m_begin + c * CP;
        constexpr int PIECES = CP / 8;          // 16-byte pieces per channel row
        constexpr int ROWS_PER = 64 / PIECES;   // rows covered by one wave-wide pass
#pragma unroll
        for (int k = 0; k < 32 / ROWS_PER; ++k) {
            const int r = k * ROWS_PER + lane / PIECES, piece = lane % PIECES;
            const u32x4 v = *(const u32x4 *)&ow[r * OROW + 8 * piece];
            const PixPos pp = advance(c0, 8 * piece, hw);
            const int co = ct * kTileCo + wave * 32 + r;
            const bool ok = live && mc + 8 * piece < m_end && co < s.C_out;
            buf_store16(yr, ok ? (uint32_t)((pp.n * s.C_out + co) * hw + pp.p) * 2u : kOOB, v);
        }
        __builtin_amdgcn_wave_barrier();  // staging reads done before the tile is rewritten
    };

    // Pipeline (PD chunks of x in flight; two accumulator sets):
    //   stage c: copy chunk c to LDS, request chunk c+PD, barrier, then run
    //   the MFMAs of chunk c interleaved with the epilogue of chunk c-1.
    // Stage 0 has no previous chunk (its epilogue stores nothing) and stage
    // n_chunks no current one (its MFMAs run on zeros and are discarded):
    // keeping both halves unconditional keeps them in one basic block, so
    // the scheduler can interleave MFMAs with the epilogue's VALU work.
    u32x4 r[PD][TASKS];
#pragma unroll
    for (int d = 0; d < PD; ++d) load_chunk(d, r[d]);

    // Weights (B operand of the 32x32x16 MFMA): lane holds channel co_lane
    // and k = 16*ks + 8*(lane>>5) .. +7; fetched after the first chunks of x
    // have been requested so that their latency overlaps the x stream.  The
    // epilogue constants are folded: v = acc*sc + bi, -v*log2(e) = acc*sn + bn.
    sc = co_lane < s.C_out ? scale[co_lane] : 0.f;
    bi = co_lane < s.C_out ? bias[co_lane] : 0.f;
    sn = sc * -1.4426950408889634f;
    bn = bi * -1.4426950408889634f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int k = 16 * ks + 8 * (lane >> 5);
        wf[ks] = (co_lane < s.C_out && k < s.C_in) ? *(const u32x4 *)(w + co_lane * s.C_in + k)
                                                   : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 acc0[MB], acc1[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc1[i][e] = 0.f;
    // The stage body for chunk c (d = c % PD is a compile-time constant).
    auto stage = [&](int c, auto dconst, f32x16 (&acc_cur)[MB], f32x16 (&acc_prev)[MB]) {
        constexpr int d = decltype(dconst)::value;
        store_chunk(c & 1, r[d]);
        load_chunk(c + PD, r[d]);
        __syncthreads();
        // Waves w and w+4 share a SIMD.  The two halves of the stage are
        // independent, so the two waves run them in opposite orders: while
        // one keeps the matrix core busy the other issues the previous
        // chunk's epilogue arithmetic, and then they swap.
        if (wave < kWaves / 2) {
            mfma_chunk(c & 1, acc_cur);
            epi_math(acc_prev);
        } else {
            epi_math(acc_prev);
            mfma_chunk(c & 1, acc_cur);
        }
        epi_store(c - 1, c > 0);
    };
    static_assert(PD % 2 == 0, "accumulator sets alternate with chunk parity");
    for (int cb = 0; cb <= n_chunks; cb += PD) {
        static_for<0, PD>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            const int c = cb + d;
            if (c > n_chunks) return;
            if constexpr (d % 2 == 0)
                stage(c, dc, acc0, acc1);
            else
                stage(c, dc, acc1, acc0);
        });
    }
}

template <int KS, int CP, int PD, int EPI>
hipError_t launch_pw(const Shape &s, const void *x, const void *w, const float *scale, const float *bias,
                     void *y, hipStream_t st, int num_cu) {
    const int co_tiles = (s.C_out + kTileCo - 1) / kTileCo;
    // One workgroup per compute unit in total, split over the channel
    // tiles; each owns a balanced run of pixels (a multiple of 8).
    int n_ranges = (num_cu + co_tiles - 1) / co_tiles;
    int px_per_wg = (s.M + n_ranges - 1) / n_ranges;
    px_per_wg = (px_per_wg + 7) / 8 * 8;
    n_ranges = (s.M + px_per_wg - 1) / px_per_wg;
    const int ranges_per_xcd = (n_ranges + 7) / 8;
    const int blocks = ranges_per_xcd * 8 * co_tiles;
    hipLaunchKernelGGL((pointwise_bf16<KS, CP, PD, EPI>), dim3(blocks), dim3(kThreadsPw), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, px_per_wg,
                       co_tiles, n_ranges, ranges_per_xcd);
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
    const int ks = (s.C_in + 15) / 16;
#define CBS_PW(KS_)                                                                              \
    if (ks <= KS_)                                                                               \
        return epi == kFused ? launch_pw<KS_, 32, 4, kFused>(s, x, w, scale, bias, y, st, num_cu) \
                             : launch_pw<KS_, 32, 4, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
    CBS_PW(4) CBS_PW(8) CBS_PW(16)
#undef CBS_PW
    return hipErrorInvalidValue;
}

}  // namespace cbs
