// k_stem.hip -- the small-K variant: a 3x3, stride-2, padding-1 layer with at
// most 3 input channels and at most 16 output channels (an RGB stem).
//
// With C_in = 3 the implicit GEMM's reduction is K = 27, which fits one
// v_mfma_f32_16x16x32_bf16 (K padded to 32 with zero weights), so each 16
// output pixels x 16 output channels cost one instruction and the layer is
// bound by streaming x in and y out ("Fusing an Epilogue", section "Three
// kernels for one operation": a GEMM tile would waste most of its columns on
// so few output channels).
//
//  * One workgroup per compute unit owns a run of output rows of one image
//    and walks it two output rows per step.
//  * Input rows are kept in LDS as a ring of 16 row slots, each holding, per
//    input channel, the row's "horizontal im2col": for tap column kw the
//    array A_kw[ow] = x[ih][2*ow + kw - 1] (zero outside the row).  Built
//    from 16-byte loads of 8 input columns, split into even and odd columns
//    with byte permutes; the kw = 0 array, shifted by one column, comes from
//    a second load 4 bytes earlier (or, at the row start, from the odd
//    columns shifted in registers).
//  * The MFMA A fragment (16 pixels x 8 consecutive k per lane group) is two
//    ds_read_b64_tr_b16 reads of four k-rows each: k = (ci, kh, kw) picks the
//    array of input row 2*oh - 1 + kh, channel ci, tap kw; k >= 9*C_in reads
//    a zero row.  The weights (B operand, 8 k values of one output channel
//    per lane) stay in 4 VGPRs.
//  * Two batches of 4 input rows are in flight in registers while a step
//    computes; one barrier per step.
//  * Epilogue (folded BN, SiLU, bf16) on the accumulators, staged per wave in
//    LDS and stored as whole 16-byte pieces of output rows.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr(const char *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

template <int B, int E, typename F>
__device__ __forceinline__ void unroll(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        unroll<B + 1, E>(f);
    }
}

constexpr int kStemWaves = 8;
constexpr int kStemThreads = 64 * kStemWaves;
constexpr int kRing = 16;  // input-row slots (a step reads 5 rows; 13 rows can be live)

// Compile-time geometry for output rows of at most 64*NBW pixels (NBW:
// 16-pixel blocks per wave per step of two rows).
template <int NBW>
struct StemGeo {
    static constexpr int OWMAX = 64 * NBW;
    static constexpr int P = 2 * OWMAX + 32;       // bytes per im2col array (padding spreads banks)
    static constexpr int SLOT = 9 * P + 64;        // bytes per input row: 3 channels x 3 taps
    static constexpr int RINGB = kRing * SLOT;     // the zero row follows the ring
    static constexpr int SP = 16 * NBW + 8;        // staging pitch (elements) per channel row
    static constexpr int MAXT = (192 * NBW + kStemThreads - 1) / kStemThreads;  // loads per batch/thread
};

template <int NBW, int EPI>
__global__ __launch_bounds__(kStemThreads, 1) void stem_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int rows_per_wg, int wg_per_image) {
    using G = StemGeo<NBW>;
    __shared__ __attribute__((aligned(16))) char ring[G::RINGB + G::P];
    __shared__ __attribute__((aligned(16))) uint16_t stg[kStemWaves][16 * G::SP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)blockIdx.x / wg_per_image;
    const int r0 = ((int)blockIdx.x % wg_per_image) * rows_per_wg;
    if (n >= s.N || r0 >= s.OH) return;  // uniform
    const int r1 = min(r0 + rows_per_wg, s.OH);
    const int steps = (r1 - r0 + 1) / 2;
    const int bpr = s.OW / 16;      // 16-pixel blocks per output row
    const int segs = s.W / 8;       // 8-column input segments per row
    const int tasks = 4 * s.C_in * segs;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.H * s.W * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);

    // Input stream: row i of the stream is input row ih = 2*r0 - 1 + i.
    // Batch b holds stream rows 4b-3 .. 4b; step t reads rows 4t .. 4t+4,
    // i.e. batches t and t+1.  A row outside the image, or past the last one
    // the workgroup reads, is not fetched (its loads return zeros).
    u32x4 ra[2][G::MAXT], rs[2][G::MAXT];
    auto load_batch = [&](int b, u32x4 (&a)[G::MAXT], u32x4 (&sh)[G::MAXT]) {
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) {
            const int t = tid + q * kStemThreads;
            const int rr = t / (s.C_in * segs), rem = t - rr * (s.C_in * segs);
            const int ci = rem / segs, seg = rem - ci * segs;
            const int i = 4 * b - 3 + rr, ih = 2 * r0 - 1 + i;
            const bool ok = t < tasks && i >= 0 && i <= 4 * steps && ih >= 0 && ih < s.H;
            const uint32_t off = (uint32_t)(((n * s.C_in + ci) * s.H + ih) * s.W + 8 * seg) * 2u;
            a[q] = buf_load16(xr, ok ? off : kOOB);
            // x[8 seg - 2 .. 8 seg + 5]: its odd columns are the kw = 0 taps.
            // Not needed at the row start (seg 0), where they come from `a`.
            sh[q] = buf_load16(xr, ok && seg > 0 ? off - 4u : kOOB);
        }
    };
    // Scatter batch b into its ring slots: per (row, channel, segment) the
    // even columns (kw = 1), odd columns (kw = 2) and the odd columns one to
    // the left (kw = 0), 4 output pixels each.
    auto write_batch = [&](int b, const u32x4 (&a)[G::MAXT], const u32x4 (&sh)[G::MAXT]) {
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) {
            const int t = tid + q * kStemThreads;
            if (t >= tasks) continue;
            const int rr = t / (s.C_in * segs), rem = t - rr * (s.C_in * segs);
            const int ci = rem / segs, seg = rem - ci * segs;
            const int i = 4 * b - 3 + rr;
            char *dst = ring + (i & (kRing - 1)) * G::SLOT + ci * 3 * G::P + 8 * seg;
            const u32x4 v = a[q], u = sh[q];
            const uint32_t e0 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
            const uint32_t e1 = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
            const uint32_t o0 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
            const uint32_t o1 = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
            uint32_t l0 = __builtin_amdgcn_perm(u.y, u.x, 0x07060302u);
            uint32_t l1 = __builtin_amdgcn_perm(u.w, u.z, 0x07060302u);
            if (seg == 0) {  // left padding, then the odd columns shifted right by one
                l0 = o0 << 16;
                l1 = __builtin_amdgcn_alignbit(o1, o0, 16);
            }
            *(u32x2 *)(dst) = u32x2{l0, l1};
            *(u32x2 *)(dst + G::P) = u32x2{e0, e1};
            *(u32x2 *)(dst + 2 * G::P) = u32x2{o0, o1};
        }
    };

    // Zero row (k >= 9*C_in and channels >= C_in read it).
    for (int i = tid; i < G::P / 16; i += kStemThreads) *(u32x4 *)(ring + G::RINGB + 16 * i) = u32x4{0, 0, 0, 0};

    load_batch(0, ra[0], rs[0]);
    load_batch(1, ra[1], rs[1]);

    // Transposed-read geometry of the 16x16x32 A operand: lane l holds pixel
    // l&15 of a block and k = 8*(l>>4) .. +7.  In read h (k = 8*(l>>4) + 4h
    // .. +3) lane j = l&15 of its group loads k-row 8*(l>>4) + 4h + (j>>2) at
    // pixels 4*(j&3) .. +3.
    const int grp = lane >> 4, jq = lane & 15;
    int kh_of[2], off_of[2];
    bool zero_of[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = 8 * grp + 4 * h + (jq >> 2);
        const int ci = k / 9, r = k - 9 * ci, kh = r / 3, kw = r - 3 * kh;
        zero_of[h] = k >= 9 * s.C_in;
        kh_of[h] = kh;
        off_of[h] = (ci * 3 + kw) * G::P + 8 * (jq & 3);
    }
    // Weights: lane l holds output channel l&15, k = 8*(l>>4) .. +7; the OIHW
    // layout of a 3x3 filter is already k = (ci*3 + kh)*3 + kw.
    const int co = lane & 15;
    const int kdim = 9 * s.C_in;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k0 = 8 * grp + 2 * e;
        const uint32_t lo = (co < s.C_out && k0 < kdim) ? w[co * kdim + k0] : 0u;
        const uint32_t hi = (co < s.C_out && k0 + 1 < kdim) ? w[co * kdim + k0 + 1] : 0u;
        wv[e] = lo | (hi << 16);
    }
    const bf16x8 wf = __builtin_bit_cast(bf16x8, u32x4{wv[0], wv[1], wv[2], wv[3]});
    const float sc = co < s.C_out ? scale[co] : 0.f, bi = co < s.C_out ? bias[co] : 0.f;
    const float sn = sc * -1.4426950408889634f, bn = bi * -1.4426950408889634f;

    write_batch(0, ra[0], rs[0]);
    load_batch(2, ra[0], rs[0]);
    write_batch(1, ra[1], rs[1]);
    load_batch(3, ra[1], rs[1]);

    uint16_t *const ow_ = stg[wave];
    auto compute = [&](int t) {
        f32x4 acc[NBW];
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            int gb = wave * NBW + bb;
            if (gb >= 2 * bpr) gb = 0;  // idle block: read valid memory, store nothing
            const int row = gb >= bpr ? 1 : 0, bx = gb - row * bpr;
            u32x2 part[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int slot = (4 * t + 2 * row + kh_of[h]) & (kRing - 1);
                const int a = zero_of[h] ? G::RINGB + 8 * (jq & 3) : slot * G::SLOT + off_of[h];
                part[h] = lds_read_tr(ring + a + 32 * bx);
            }
            const bf16x8 af = __builtin_bit_cast(bf16x8, u32x4{part[0].x, part[0].y, part[1].x, part[1].y});
            acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
        // Epilogue: lane holds channel co, pixels 4*grp .. +3 of each block.
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = acc[bb][r];
                if (EPI == kFused) {
                    const float v = __builtin_fmaf(a, sc, bi);
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(a, sn, bn));
                    o[r] = v * __builtin_amdgcn_rcpf(1.0f + e);
                } else {
                    o[r] = a;
                }
            }
            *(u32x2 *)&ow_[co * G::SP + 16 * bb + 4 * grp] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staging writes done
        __builtin_amdgcn_wave_barrier();
        // Store: 16 channel rows x 2*NBW pieces of 8 pixels.
#pragma unroll
        for (int it = 0; it < (2 * 16 * NBW + 63) / 64; ++it) {
            const int p = it * 64 + lane;
            const int c = p / (2 * NBW), pc = p - c * (2 * NBW);
            const int bb = pc >> 1, half = pc & 1;
            const int gb = wave * NBW + bb;
            const int row = gb >= bpr ? 1 : 0, bx = gb - row * bpr;
            const int oh = r0 + 2 * t + row;
            const bool ok = p < 32 * NBW && gb < 2 * bpr && oh < r1 && c < s.C_out;
            const u32x4 v = *(const u32x4 *)&ow_[(ok ? c : 0) * G::SP + 16 * bb + 8 * half];
            const uint32_t off = (uint32_t)(((n * s.C_out + c) * s.OH + oh) * s.OW + 16 * bx + 8 * half) * 2u;
            buf_store16(yr, ok ? off : kOOB, v);
        }
        __builtin_amdgcn_wave_barrier();
    };

    // Step t: scatter batch t+2 (loaded two steps ago), request batch t+4,
    // barrier (batch t+1 visible; slots of rows read two steps ago free),
    // then compute output rows r0+2t, r0+2t+1.
    for (int t = 0; t < steps; t += 2) {
        unroll<0, 2>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            const int tt = t + d;
            if (tt >= steps) return;
            write_batch(tt + 2, ra[d], rs[d]);
            load_batch(tt + 4, ra[d], rs[d]);
            __syncthreads();
            compute(tt);
        });
    }
}

template <int NBW, int EPI>
hipError_t launch_stem_t(const Shape &s, const void *x, const void *w, const float *scale, const float *bias,
                         void *y, hipStream_t st, int num_cu) {
    // About one workgroup per compute unit: split each image's output rows
    // into wg_per_image runs of an even number of rows.
    int wg_per_image = num_cu / s.N;
    if (wg_per_image < 1) wg_per_image = 1;
    if (wg_per_image > (s.OH + 1) / 2) wg_per_image = (s.OH + 1) / 2;
    int rows = (s.OH + wg_per_image - 1) / wg_per_image;
    rows = (rows + 1) & ~1;
    wg_per_image = (s.OH + rows - 1) / rows;
    hipLaunchKernelGGL((stem_bf16<NBW, EPI>), dim3(s.N * wg_per_image), dim3(kStemThreads), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, rows,
                       wg_per_image);
    return hipGetLastError();
}

}  // namespace

bool stem_supports(const Shape &s, int dtype) {
    return dtype == kDtypeBf16 && s.KH == 3 && s.KW == 3 && s.stride == 2 && s.pad == 1 && s.C_in <= 3 &&
           s.C_out <= 16 && s.W % 32 == 0 && s.OW == s.W / 2 && s.OW <= StemGeo<5>::OWMAX &&
           (uint64_t)s.N * s.C_in * s.H * s.W * 2 <= kMaxBufferBytes &&
           (uint64_t)s.N * s.C_out * s.OHW * 2 <= kMaxBufferBytes;
}

bool stem_pointers_ok(const void *x, const void *w, const void *y) {
    return (((uintptr_t)x | (uintptr_t)y) & 15) == 0 && ((uintptr_t)w & 1) == 0;
}

hipError_t launch_stem(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                       const float *bias, void *y, hipStream_t st, int num_cu) {
#define CBS_STEM(NBW_)                                                                                \
    if (s.OW <= StemGeo<NBW_>::OWMAX)                                                                 \
        return epi == kFused ? launch_stem_t<NBW_, kFused>(s, x, w, scale, bias, y, st, num_cu)       \
                             : launch_stem_t<NBW_, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
    CBS_STEM(1) CBS_STEM(2) CBS_STEM(5)
#undef CBS_STEM
    return hipErrorInvalidValue;
}

}  // namespace cbs
