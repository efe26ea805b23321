// k_gather.hip -- implicit-GEMM convolution on MFMA, generic over every shape.
//
// "Convolution as a GEMM" (page "Fusing an Epilogue", section "Three kernels
// for one operation"): rows are output pixels m = (n*OH + oh)*OW + ow, columns
// are output channels, and the reduction runs over k = (ci*KH + kh)*KW + kw.
// No im2col matrix is materialised: every 32-wide k slice of the pixel
// operand is gathered straight from NCHW x into LDS (zeros for padding and for
// the ragged K and M tails), the weight slice is copied from OIHW w, and the
// K loop accumulates one tile product per k slice, as in the tiled loop of
// section "The shape of it".
// After the loop the tile is still in registers and the epilogue applies the
// folded batch norm and SiLU before the single store.
//
// This is the variant of last resort: it serves any geometry and both dtypes,
// with double-buffered LDS slices and one barrier per slice, but each pixel's
// k values are fetched one element at a time.  The window and pointwise
// variants replace it on the shapes they serve.
#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

constexpr int kThreads = 256;  // 4 waves of 64, arranged 2 (pixels) x 2 (channels)
constexpr int kBM = 128;       // output pixels per workgroup tile
constexpr int kBN = 64;        // output channels per workgroup tile

// ---------------------------------------------------------------- bf16 -----
// LDS rows hold one pixel (or channel) x 32 k values, padded to 40 elements
// (80 bytes) so that the 16-byte fragment reads of 8 consecutive rows fall in
// distinct bank groups.
constexpr int kBK16 = 32;
constexpr int kLd16 = 40;

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_gather_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const float *__restrict__ scale, const float *__restrict__ bias,
    uint16_t *__restrict__ y, Shape s) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLd16];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLd16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_tiles = (s.C_out + kBN - 1) / kBN;
    const int m0 = (int)(blockIdx.x / n_tiles) * kBM;
    const int co0 = (int)(blockIdx.x % n_tiles) * kBN;

    // Gather role: one pixel, 16 of the 32 k values of each slice.
    const int a_px = tid & (kBM - 1), a_half = tid >> 7;
    const int am = m0 + a_px;
    const bool am_ok = am < s.M;
    int an = 0, aih0 = 0, aiw0 = 0;
    if (am_ok) {
        an = am / s.OHW;
        const int r = am - an * s.OHW;
        const int oh = r / s.OW, ow = r - (r / s.OW) * s.OW;
        aih0 = oh * s.stride - s.pad;
        aiw0 = ow * s.stride - s.pad;
    }
    const uint16_t *xn = x + (size_t)an * s.C_in * s.HW;
    // Weight role: one output channel, 8 consecutive k values.
    const int b_co = tid >> 2, b_kq = (tid & 3) * 8;
    const bool b_ok = co0 + b_co < s.C_out;
    const uint16_t *wrow = w + (size_t)(b_ok ? co0 + b_co : 0) * s.K;

    uint16_t ra[16], rb[8];
    auto load_slice = [&](int k0) {
        int k = k0 + 16 * a_half;
        int ci = k / s.T;
        const int rr = k - ci * s.T;
        int kh = rr / s.KW, kw = rr - (rr / s.KW) * s.KW;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int ih = aih0 + kh, iw = aiw0 + kw;
            const bool ok = am_ok && (k + j) < s.K && (unsigned)ih < (unsigned)s.H &&
                            (unsigned)iw < (unsigned)s.W;
            ra[j] = ok ? xn[ci * s.HW + ih * s.W + iw] : (uint16_t)0;
            if (++kw == s.KW) {
                kw = 0;
                if (++kh == s.KH) { kh = 0; ++ci; }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = k0 + b_kq + j;
            rb[j] = (b_ok && kk < s.K) ? wrow[kk] : (uint16_t)0;
        }
    };
    auto store_slice = [&](int buf) {
        u32x4 a0, a1, b0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a0[j] = (uint32_t)ra[2 * j] | ((uint32_t)ra[2 * j + 1] << 16);
            a1[j] = (uint32_t)ra[8 + 2 * j] | ((uint32_t)ra[8 + 2 * j + 1] << 16);
            b0[j] = (uint32_t)rb[2 * j] | ((uint32_t)rb[2 * j + 1] << 16);
        }
        *(u32x4 *)&As[buf][a_px * kLd16 + 16 * a_half] = a0;
        *(u32x4 *)&As[buf][a_px * kLd16 + 16 * a_half + 8] = a1;
        *(u32x4 *)&Bs[buf][b_co * kLd16 + b_kq] = b0;
    };

    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_slices = (s.K + kBK16 - 1) / kBK16;
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int sl = 0; sl < n_slices; ++sl) {
        const int buf = sl & 1;
        if (sl + 1 < n_slices) load_slice((sl + 1) * kBK16);
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *(const bf16x8 *)&As[buf][(wm * 64 + i * 16 + lr) * kLd16 + lg * 8];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[j] = *(const bf16x8 *)&Bs[buf][(wn * 32 + j * 16 + lr) * kLd16 + lg * 8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        if (sl + 1 < n_slices) store_slice(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds channel co = lr of each 16x16 block and pixels
    // 4*lg .. 4*lg+3 of it.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int co = co0 + wn * 32 + j * 16 + lr;
        if (co >= s.C_out) continue;
        float sc = 1.f, bi = 0.f;
        if (EPI == kFused) { sc = scale[co]; bi = bias[co]; }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + lg * 4 + r;
                if (m >= s.M) continue;
                const int n = m / s.OHW, rem = m - (m / s.OHW) * s.OHW;
                const float v = acc[i][j][r];
                const float o = (EPI == kFused) ? bn_silu(v, sc, bi) : v;
                y[(n * s.C_out + co) * s.OHW + rem] = to_bf16(o);
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 -----
// Same structure on v_mfma_f32_16x16x4_f32: 16-wide k slices, LDS rows of 16
// floats padded to 20 (80 bytes).  Each lane reads 4 consecutive k of its row
// and feeds them to 4 MFMAs; A and B use the same k order, so the sum is the
// full reduction.
constexpr int kBK32 = 16;
constexpr int kLd32 = 20;

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_gather_f32(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ scale, const float *__restrict__ bias,
    float *__restrict__ y, Shape s) {
    __shared__ __attribute__((aligned(16))) float As[2][kBM * kLd32];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBN * kLd32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_tiles = (s.C_out + kBN - 1) / kBN;
    const int m0 = (int)(blockIdx.x / n_tiles) * kBM;
    const int co0 = (int)(blockIdx.x % n_tiles) * kBN;

    const int a_px = tid & (kBM - 1), a_half = tid >> 7;
    const int am = m0 + a_px;
    const bool am_ok = am < s.M;
    int an = 0, aih0 = 0, aiw0 = 0;
    if (am_ok) {
        an = am / s.OHW;
        const int r = am - an * s.OHW;
        const int oh = r / s.OW, ow = r - (r / s.OW) * s.OW;
        aih0 = oh * s.stride - s.pad;
        aiw0 = ow * s.stride - s.pad;
    }
    const float *xn = x + (size_t)an * s.C_in * s.HW;
    const int b_co = tid >> 2, b_kq = (tid & 3) * 4;
    const bool b_ok = co0 + b_co < s.C_out;
    const float *wrow = w + (size_t)(b_ok ? co0 + b_co : 0) * s.K;

    float ra[8], rb[4];
    auto load_slice = [&](int k0) {
        int k = k0 + 8 * a_half;
        int ci = k / s.T;
        const int rr = k - ci * s.T;
        int kh = rr / s.KW, kw = rr - (rr / s.KW) * s.KW;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ih = aih0 + kh, iw = aiw0 + kw;
            const bool ok = am_ok && (k + j) < s.K && (unsigned)ih < (unsigned)s.H &&
                            (unsigned)iw < (unsigned)s.W;
            ra[j] = ok ? xn[ci * s.HW + ih * s.W + iw] : 0.f;
            if (++kw == s.KW) {
                kw = 0;
                if (++kh == s.KH) { kh = 0; ++ci; }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = k0 + b_kq + j;
            rb[j] = (b_ok && kk < s.K) ? wrow[kk] : 0.f;
        }
    };
    auto store_slice = [&](int buf) {
        *(f32x4 *)&As[buf][a_px * kLd32 + 8 * a_half] = f32x4{ra[0], ra[1], ra[2], ra[3]};
        *(f32x4 *)&As[buf][a_px * kLd32 + 8 * a_half + 4] = f32x4{ra[4], ra[5], ra[6], ra[7]};
        *(f32x4 *)&Bs[buf][b_co * kLd32 + b_kq] = f32x4{rb[0], rb[1], rb[2], rb[3]};
    };

    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_slices = (s.K + kBK32 - 1) / kBK32;
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int sl = 0; sl < n_slices; ++sl) {
        const int buf = sl & 1;
        if (sl + 1 < n_slices) load_slice((sl + 1) * kBK32);
        f32x4 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *(const f32x4 *)&As[buf][(wm * 64 + i * 16 + lr) * kLd32 + lg * 4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[j] = *(const f32x4 *)&Bs[buf][(wn * 32 + j * 16 + lr) * kLd32 + lg * 4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][q], bfr[j][q], acc[i][j], 0, 0, 0);
        if (sl + 1 < n_slices) store_slice(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int co = co0 + wn * 32 + j * 16 + lr;
        if (co >= s.C_out) continue;
        float sc = 1.f, bi = 0.f;
        if (EPI == kFused) { sc = scale[co]; bi = bias[co]; }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + lg * 4 + r;
                if (m >= s.M) continue;
                const int n = m / s.OHW, rem = m - (m / s.OHW) * s.OHW;
                const float v = acc[i][j][r];
                y[(n * s.C_out + co) * s.OHW + rem] = (EPI == kFused) ? bn_silu(v, sc, bi) : v;
            }
        }
    }
}

}  // namespace

bool gemm_gather_supports(const Shape &, int) { return true; }

hipError_t launch_gemm_gather(const Shape &s, int dtype, int epi, const void *x, const void *w,
                              const float *scale, const float *bias, void *y, hipStream_t st) {
    const unsigned m_tiles = (unsigned)((s.M + kBM - 1) / kBM);
    const unsigned n_tiles = (unsigned)((s.C_out + kBN - 1) / kBN);
    const dim3 grid(m_tiles * n_tiles), block(kThreads);
    if (dtype == kDtypeBf16) {
        auto xx = (const uint16_t *)x;
        auto ww = (const uint16_t *)w;
        auto yy = (uint16_t *)y;
        if (epi == kFused)
            hipLaunchKernelGGL(gemm_gather_bf16<kFused>, grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else
            hipLaunchKernelGGL(gemm_gather_bf16<kConvOnly>, grid, block, 0, st, xx, ww, scale, bias, yy, s);
    } else {
        auto xx = (const float *)x;
        auto ww = (const float *)w;
        auto yy = (float *)y;
        if (epi == kFused)
            hipLaunchKernelGGL(gemm_gather_f32<kFused>, grid, block, 0, st, xx, ww, scale, bias, yy, s);
        else
            hipLaunchKernelGGL(gemm_gather_f32<kConvOnly>, grid, block, 0, st, xx, ww, scale, bias, yy, s);
    }
    return hipGetLastError();
}

}  // namespace cbs
