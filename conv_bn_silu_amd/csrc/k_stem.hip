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
//  * Workgroups of 4 waves, two per compute unit (their LDS fits twice), so
//    one workgroup's loads and stores overlap the other's arithmetic.  Each
//    computes one output row per step.  The G workgroups interleave over the
//    N*OH output rows (workgroup j takes rows j, j+G, j+2G, ...), so at any
//    time the whole chip reads and writes one contiguous window of x and y:
//    DRAM pages stay open, which is worth about 10% of the bandwidth here
//    over giving each workgroup its own run of rows.  The eight XCDs take
//    contiguous slices of each window, so an input row shared by two
//    neighbouring output rows is fetched into one L2.
//  * The 3 input rows of a step are kept in LDS (3 sets of 3 row slots: the
//    step being computed, the next being written, and the previous one that
//    a slower wave may still read), each holding, per input channel, the
//    row's "horizontal im2col": for tap column kw the
//    array A_kw[ow] = x[ih][2*ow + kw - 1] (zero outside the row).  Built
//    from 16-byte loads of 8 input columns, split into even and odd columns
//    with byte permutes; the kw = 0 array is the odd columns shifted by one,
//    whose first element comes from the lane holding the previous 8 columns:
//    a wave-wide load covers 63 new segments in lanes 1..63 and repeats the
//    one before them in lane 0, and each lane takes the column from the
//    lane below by a DPP wave shift.
//  * The MFMA A fragment (16 pixels x 8 consecutive k per lane group) is two
//    ds_read_b64_tr_b16 reads of four k-rows each: k = (ci, kh, kw) picks the
//    array of input row 2*oh - 1 + kh, channel ci, tap kw; k >= 9*C_in reads
//    a zero row.  The weights (B operand, 8 k values of one output channel
//    per lane) stay in 4 VGPRs.
//  * A step's input rows are loaded kStemPD steps ahead into registers; one
//    barrier per step.
//  * Epilogue (folded BN, SiLU, bf16) on the accumulators, staged by all four
//    waves in one LDS copy of the step's output row (16 channel rows, double
//    buffered) and stored after the next step's barrier by the whole
//    workgroup: four consecutive lanes write one 64-byte segment of a channel
//    row, with the streaming cache policy where OW is a multiple of 32 (each
//    wave storing its own 80-pixel slices split segments between waves:
//    41.0 -> 38.5 us on the stem layer at N=32, 640x640, same bits).
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

constexpr int kStemWaves = 4;
constexpr int kStemThreads = 64 * kStemWaves;
constexpr int kStemPD = 3;  // steps of input rows in flight in registers (>= 1; 3 measured fastest)
constexpr int kRing = 9;    // input-row slots: 3 steps x 3 rows (see the step loop)

// Compile-time geometry for output rows of at most 64*NBW pixels (NBW:
// 16-pixel blocks per wave per output row).
template <int NBW>
struct StemGeo {
    static constexpr int OWMAX = 16 * kStemWaves * NBW;
    static constexpr int P = 2 * OWMAX + 32;   // bytes per im2col array (padding spreads banks)
    static constexpr int SLOT = 9 * P + 64;    // bytes per input row: 3 channels x 3 taps
    static constexpr int RINGB = kRing * SLOT; // the zero row follows the ring
    // Output staging pitch (elements) per channel row: 2 SPW bytes is an odd
    // multiple of 16, so the 8-byte staging writes of 16 channels x 2 lane
    // groups (one 32-lane pass) cover all 64 banks.
    static constexpr int SPW = OWMAX + 8;
    // 16-byte copy tasks per thread per step: 3 rows x 3 channels x W/8,
    // 63 new ones per wave-wide load.
    static constexpr int MAXT = ((3 * 3 * (2 * OWMAX / 8) + 62) / 63 + kStemWaves - 1) / kStemWaves;
};

template <int NBW, int EPI>
__global__ __launch_bounds__(kStemThreads, 2) void stem_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int wg_per_xcd) {
    using G = StemGeo<NBW>;
    __shared__ __attribute__((aligned(16))) char ring[G::RINGB + G::P];
    __shared__ __attribute__((aligned(16))) uint16_t stg[2][16 * G::SPW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Block -> rank j among the G = 8*wg_per_xcd workgroups: XCD x (= block
    // id mod 8) holds ranks x*wg_per_xcd .. +wg_per_xcd-1.  Step t computes
    // global output row j + t*G (image n = row / OH, row oh = row mod OH).
    const int gsz = 8 * wg_per_xcd;
    const int j = ((int)blockIdx.x & 7) * wg_per_xcd + ((int)blockIdx.x >> 3);
    const int rows_total = s.N * s.OH;
    if (j >= rows_total) return;  // uniform
    const int steps = (rows_total - j + gsz - 1) / gsz;
    const int bpr = s.OW / 16;      // 16-pixel blocks per output row
    const int segs = s.W / 8;       // 8-column input segments per row
    const int tasks = 3 * s.C_in * segs;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.H * s.W * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);

    // Copy task q of this thread, task index t = 63 (4 q + wave) + lane - 1,
    // is (input row kh of the step -- input row 2*oh - 1 + kh --, channel
    // ci, 8-column segment seg).  Its place in x and in LDS is fixed but for
    // the step.  Consecutive lanes hold consecutive segments of one row
    // unless seg == 0; lane 0 holds the segment before lane 1's and is only
    // loaded.
    int tk_rr[G::MAXT], tk_lds[G::MAXT];
    uint32_t tk_goff[G::MAXT];
    bool tk_load[G::MAXT], tk_valid[G::MAXT], tk_first[G::MAXT];
#pragma unroll
    for (int q = 0; q < G::MAXT; ++q) {
        const int traw = 63 * (q * kStemWaves + wave) + lane - 1;
        const int t = traw < 0 ? 0 : traw;
        const int rr = t / (s.C_in * segs), rem = t - rr * (s.C_in * segs);
        const int ci = rem / segs, seg = rem - ci * segs;
        tk_load[q] = traw >= 0 && t < tasks;
        tk_valid[q] = lane > 0 && t < tasks;
        tk_first[q] = seg == 0;
        tk_rr[q] = rr;
        tk_goff[q] = (uint32_t)((ci * s.H + rr) * s.W + 8 * seg) * 2u;
        tk_lds[q] = rr * G::SLOT + ci * 3 * G::P + 8 * seg;
    }

    // ra: x[8 seg .. 8 seg + 7].
    u32x4 ra[kStemPD][G::MAXT];
    auto load_step = [&](int t, u32x4 (&a)[G::MAXT]) {
        const int row = j + t * gsz;  // uniform
        const int nn = row / s.OH, oh = row - nn * s.OH;
        const bool live = t < steps;
        // First input row of the step, 2*oh - 1, relative to the image.
        const int ih0 = 2 * oh - 1;
        const uint32_t base = (uint32_t)((nn * s.C_in * s.H + ih0) * s.W) * 2u;
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) {
            const int ih = ih0 + tk_rr[q];
            const bool ok = live && tk_load[q] && (uint32_t)ih < (uint32_t)s.H;
            a[q] = buf_load16(xr, ok ? base + tk_goff[q] : kOOB);
        }
    };
    // Scatter step t's rows into its slot set: per (row, channel, segment)
    // the even columns (kw = 1), odd columns (kw = 2) and the odd columns one
    // to the left (kw = 0), 4 output pixels each.
    auto write_step = [&](int t, const u32x4 (&a)[G::MAXT]) {
        char *const set = ring + (t % 3) * 3 * G::SLOT;
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) {
            const u32x4 v = a[q];
            const uint32_t e0 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
            const uint32_t e1 = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
            const uint32_t o0 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
            const uint32_t o1 = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
            // Column 8 seg - 1 sits in the upper half of the o1 of the lane
            // below (wave_shr:1); zero at the row start.
            uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o1, 0x138, 0xf, 0xf, false);
            prev = tk_first[q] ? 0u : prev;
            if (!tk_valid[q]) continue;
            char *dst = set + tk_lds[q];
            const uint32_t l0 = __builtin_amdgcn_perm(o0, prev, 0x05040302u);
            const uint32_t l1 = __builtin_amdgcn_alignbit(o1, o0, 16);
            *(u32x2 *)(dst) = u32x2{l0, l1};
            *(u32x2 *)(dst + G::P) = u32x2{e0, e1};
            *(u32x2 *)(dst + 2 * G::P) = u32x2{o0, o1};
        }
    };

    // Zero row (k >= 9*C_in reads it).
    for (int i = tid; i < G::P / 16; i += kStemThreads) *(u32x4 *)(ring + G::RINGB + 16 * i) = u32x4{0, 0, 0, 0};

    unroll<0, kStemPD>([&](auto bc) {
        constexpr int b = decltype(bc)::value;
        load_step(b, ra[b]);
    });

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

    write_step(0, ra[0]);
    load_step(kStemPD, ra[0]);

    // This wave's blocks: block gb = wave*NBW + bb of a row starts at column
    // 16*gb; blocks past bpr are idle (they read block 0, store nothing).
    int blk_col[NBW];
#pragma unroll
    for (int bb = 0; bb < NBW; ++bb) {
        const int gb = wave * NBW + bb;
        blk_col[bb] = gb < bpr ? 32 * gb : 0;  // byte offset in an im2col array
    }
    // Store pieces of a step (output row): C_out channel rows x OW/8 pieces
    // of 8 pixels, piece p = tid + 256 it, so four consecutive lanes write 64
    // contiguous bytes of one channel row.  LDS source and offset within the
    // image's output (kOOB past C_out) are fixed; the image and row change per
    // step.
    const int ppr = s.OW >> 3;
    constexpr int kStoreIt = (16 * (G::OWMAX / 8) + kStemThreads - 1) / kStemThreads;
    uint32_t st_off[kStoreIt];
    int st_lds[kStoreIt];
#pragma unroll
    for (int it = 0; it < kStoreIt; ++it) {
        const int p = it * kStemThreads + tid;
        const int c = p / ppr, pc = p - c * ppr;
        const bool ok = c < s.C_out;
        st_lds[it] = (ok ? c : 0) * G::SPW + 8 * pc;
        st_off[it] = ok ? (uint32_t)(c * s.OHW + 8 * pc) * 2u : kOOB;
    }
    // With OW a multiple of 32 those 64 bytes are one whole aligned segment
    // of y, and the stores take the streaming policy.
    const bool whole_segments = (s.OW & 31) == 0;
    auto store_step = [&](int t) {
        const uint16_t *src = stg[t & 1];
        const int row = j + t * gsz;
        const int nn = row / s.OH, oh = row - nn * s.OH;
        const uint32_t obase = (uint32_t)((nn * s.C_out * s.OH + oh) * s.OW) * 2u;
#pragma unroll
        for (int it = 0; it < kStoreIt; ++it) {
            const u32x4 v = *(const u32x4 *)&src[st_lds[it]];
            const uint32_t off = st_off[it] == kOOB ? kOOB : obase + st_off[it];
            if (whole_segments) buf_store16_nt(yr, off, v);
            else buf_store16(yr, off, v);
        }
    };

    auto compute = [&](int t) {
        // Byte address of this lane's k-row for read h, before the block's
        // column offset.
        int base[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            base[h] = zero_of[h] ? G::RINGB + 8 * (jq & 3) : ((t % 3) * 3 + kh_of[h]) * G::SLOT + off_of[h];
        f32x4 acc[NBW];
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            const u32x2 lo = lds_read_tr(ring + base[0] + blk_col[bb]);
            const u32x2 hi = lds_read_tr(ring + base[1] + blk_col[bb]);
            const bf16x8 af = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
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
            // Staged at the block's columns of the step's output row (an idle
            // block's columns lie past OW and are never stored).
            *(u32x2 *)&stg[t & 1][co * G::SPW + 16 * (wave * NBW + bb) + 4 * grp] =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
    };

    // Step t: barrier (step t's rows, written last step, and output row t-1,
    // staged by every wave last step, become visible), then store output row
    // t-1, scatter step t+1's rows (loaded kStemPD steps earlier) into slot
    // set (t+1) mod 3, request step t+1+kStemPD's rows into the freed
    // registers and compute output row j + t*G into staging buffer t mod 2,
    // so the scatter and the stores run beside the step's arithmetic.  The
    // slot set written here was last read in step t-2, and staging buffer
    // t mod 2 in step t-1 (storing row t-2), both finished by every wave
    // before this step's barrier.
    for (int t0 = 0; t0 < steps; t0 += kStemPD) {
        unroll<0, kStemPD>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            constexpr int slot = (d + 1) % kStemPD;
            const int t = t0 + d;
            if (t >= steps) return;
            __syncthreads();
            if (t > 0) store_step(t - 1);
            write_step(t + 1, ra[slot]);
            load_step(t + 1 + kStemPD, ra[slot]);
            compute(t);
        });
    }
    __syncthreads();
    store_step(steps - 1);
}

template <int NBW, int EPI>
hipError_t launch_stem_t(const Shape &s, const void *x, const void *w, const float *scale, const float *bias,
                         void *y, hipStream_t st, int num_cu) {
    // Two workgroups per compute unit (fewer if there are fewer rows).
    const int rows_total = s.N * s.OH;
    int wgs = 2 * num_cu;
    if (wgs > rows_total) wgs = rows_total;
    const int wg_per_xcd = (wgs + 7) / 8;
    hipLaunchKernelGGL((stem_bf16<NBW, EPI>), dim3(8 * wg_per_xcd), dim3(kStemThreads), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, wg_per_xcd);
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
