// k_pointwise.hip -- the 1x1 (stride 1, no padding) layer as a streaming GEMM.
//
// For a 1x1 convolution the implicit GEMM has no window: row m of the pixel
// operand is x[n][:][p] with m = n*H*W + p, so "read x once, write y once"
// (page "Fusing an Epilogue", section "The problem") means streaming x and y
// through the chip exactly once.  How the chip walks the NCHW planes decides
// the rate: a workgroup that takes a few pixels of all channels at a time
// reads many short pieces of every plane at once, which caps DRAM at well
// under the rate of a linear copy.  So here:
//
//  * A workgroup (8 waves, two per SIMD) owns a contiguous range of L <= 224
//    pixels (at most one image boundary inside) and a tile of 256 output
//    channels, and keeps the whole [L x 256] result in accumulators: wave w
//    holds channels 32w .. 32w+31 for 7 blocks of 32 pixels.  It sweeps the
//    input channels in blocks of 32, reading 2L contiguous bytes of each
//    plane; the workgroups of one XCD hold neighbouring ranges.
//  * The weight tile (256 channels x C_in) is staged once in LDS; per block
//    of 32 input channels each lane reads its two B fragments (16 bytes
//    each) into registers.
//  * x blocks are loaded with 16-byte loads (8 pixels of one channel) two
//    blocks ahead, and stored unchanged to LDS as [channel][pixel] rows with
//    a pitch of 448 bytes (an odd multiple of 64); the A fragments (8
//    consecutive channels of one pixel per lane) come out of
//    ds_read_b64_tr_b16, whose four rows per 16-lane group then fall in
//    distinct bank quarters.
//  * v_mfma_f32_32x32x16_bf16: per block of 32 channels a wave runs 2 x 7
//    of them, with the fragment reads issued ahead.
//  * The epilogue (folded BN, SiLU, bf16 rounding) runs on the accumulators
//    one 32-pixel block at a time: the block is staged in LDS and stored as
//    16-byte pieces along its 32 channel rows before the next block is
//    computed, so the stores drain beside the epilogue's arithmetic (measured
//    1.1 us faster on the 1x1 layer at N=8, 256 -> 256, 80x80 than finishing
//    every block first).  Where the block's 64 bytes of a channel row are a
//    whole aligned segment of y, the stores use the non-temporal policy
//    (measured on the same layer: 17.5 -> 14.6 us, same bits).
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr(const unsigned char *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

constexpr int kWaves = 8;
constexpr int kThreadsPw = 64 * kWaves;
constexpr int kTileCo = 32 * kWaves;    // output channels per workgroup
constexpr int kMB = 7;                  // 32-pixel blocks per range
constexpr int kMaxL = 32 * kMB;         // pixels per range at most
constexpr int kPitch = 2 * kMaxL;       // LDS bytes per channel row (448 = 7 x 64)
constexpr int kBK = 32;                 // input channels per block
constexpr int kPieces = kBK * kMaxL / 8;  // 16-byte pieces of a block at most
constexpr int kTPT = (kPieces + kThreadsPw - 1) / kThreadsPw;  // pieces per thread
constexpr int kDepth = 4;               // fragment reads ahead of the MFMAs
constexpr int kPD = 2;                  // channel blocks in flight in registers
constexpr int kEpiPitch = 2 * kMaxL + 16;  // output staging: bytes per channel row (464)
constexpr int kEpiBytes = kWaves * 32 * kEpiPitch;

// KS: 16-channel slices of C_in (C_in <= 16*KS); PD: channel blocks in flight.
template <int KS, int PD, int EPI>
__global__ __launch_bounds__(kThreadsPw, 1) void pointwise_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int L, int n_ranges, int co_tiles) {
    constexpr int NB = (KS + 1) / 2;  // channel blocks
    constexpr int KP = 16 * KS;       // weight row length (channels, zero past C_in)
    constexpr int OCT = KP / 8;       // 16-byte octets per weight row
    constexpr int SW = (OCT < 16 ? OCT : 16) - 1;  // octet swizzle mask
    constexpr int WB = kTileCo * KP * 2;
    constexpr int AB = WB > kEpiBytes ? WB : kEpiBytes;
    // Region A holds the weight tile during the sweep and the output tile
    // for the epilogue; region B the two x block buffers.
    __shared__ __attribute__((aligned(16))) unsigned char wsm[AB];
    __shared__ __attribute__((aligned(16))) unsigned char xs[2][kBK * kPitch];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    // XCD-aware placement: XCD = block id mod 8; each XCD runs a contiguous
    // run of (range, channel tile) work items, so neighbouring ranges share
    // its L2 and the chip reads each plane as a few contiguous fronts.
    const int items = n_ranges * co_tiles;
    const int xcd = (int)blockIdx.x & 7, q8 = items >> 3, r8 = items & 7;
    const int item = xcd * q8 + min(xcd, r8) + ((int)blockIdx.x >> 3);
    if (item >= items) return;  // uniform
    const int rg = item / co_tiles, ct = item - rg * co_tiles;
    const int hw = s.HW;
    const int m0 = rg * L;
    const int len = min(L, s.M - m0);          // pixels of this range (a multiple of 8)
    const int n0 = m0 / hw, p0 = m0 - n0 * hw;  // L <= H*W: at most one image boundary inside
    auto pix = [&](int off, int &n, int &p) {  // pixel m0 + off as (image, offset)
        p = p0 + off;
        n = n0;
        if (p >= hw) {
            p -= hw;
            ++n;
        }
    };

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * hw * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * hw * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)s.C_out * s.C_in * 2u);

    // Piece t of a block (t = tid + 512 q < 32 * L/8): channel row t / (L/8),
    // pixels 8 (t mod L/8) .. +7.  Out of range (past C_in, or an idle
    // piece): an out-of-range offset, which loads zeros.
    const int qpr = len >> 3;  // pieces per row
    uint32_t pc_off[kTPT];     // byte offset of piece q at channel 0
    int pc_row[kTPT], pc_lds[kTPT];
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
        const int t = tid + q * kThreadsPw;
        const int row = t / qpr, col = t - row * qpr;
        int n, p;
        pix(8 * col, n, p);
        pc_row[q] = t < kBK * qpr ? row : kBK;  // kBK: idle
        pc_off[q] = (uint32_t)((n * s.C_in + row) * hw + p) * 2u;
        pc_lds[q] = row * kPitch + col * 16;
    }
    auto load_block = [&](int b, u32x4 (&r)[kTPT]) {
#pragma unroll
        for (int q = 0; q < kTPT; ++q) {
            const int ci = b * kBK + pc_row[q];
            const bool ok = pc_row[q] < kBK && ci < s.C_in;
            r[q] = buf_load16(xr, ok ? pc_off[q] + (uint32_t)(b * kBK * hw) * 2u : kOOB);
        }
    };
    auto store_block = [&](unsigned char *buf, const u32x4 (&r)[kTPT]) {
#pragma unroll
        for (int q = 0; q < kTPT; ++q)
            if (pc_row[q] < kBK) *(u32x4 *)(buf + pc_lds[q]) = r[q];
    };

    // The weight tile (256 channels x KP) goes to LDS once, read with
    // coalesced 16-byte loads (octet t of the tile: row t / OCT, octet
    // t mod OCT; a wave reads 1 KB contiguous) and stored at slot
    // row * OCT + (octet ^ (row & SW)): the 16 rows that a half-wave's B
    // fragment read touches then sit in 16 distinct bank groups.  (Loading
    // each lane's own fragments from global memory instead fetches each
    // cache line several times over and costs more than streaming x.)
    const int co = ct * kTileCo + wave * 32 + l32;
    {
        // Every workgroup reads the same tile at the same moment; each starts
        // at its own 1 KiB-aligned point of it (a rotation by the block id),
        // so that the requests spread over L2 channels instead of all
        // meeting on the same lines (the 1x1 layer at N=8, 256 -> 256, 80x80:
        // 14.9 -> 14.7 us, same bits).
        constexpr int NW = kTileCo * OCT / kThreadsPw;  // octets per thread
        constexpr int TOT = kTileCo * OCT;
        const int rot = (int)(((unsigned)blockIdx.x * 37u) % (unsigned)(TOT / 64)) * 64;
        u32x4 wv[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int t = (tid + i * kThreadsPw + rot) % TOT, r = t / OCT, o = t % OCT;
            const int c = ct * kTileCo + r;
            wv[i] = buf_load16(wr, (c < s.C_out && 8 * o < s.C_in) ? (uint32_t)(c * s.C_in + 8 * o) * 2u : kOOB);
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int t = (tid + i * kThreadsPw + rot) % TOT, r = t / OCT, o = t % OCT;
            *(u32x4 *)(wsm + (r * OCT + (o ^ (r & SW))) * 16) = wv[i];
        }
    }
    const int wrow = wave * 32 + l32;  // this lane's row of the weight tile
    u32x4 xr_[PD][kTPT];
#pragma unroll
    for (int d = 0; d < PD && d < NB; ++d) load_block(d, xr_[d]);
    const float sc = co < s.C_out ? scale[co] : 0.f;
    const float bi = co < s.C_out ? bias[co] : 0.f;

    f32x16 acc[kMB];
#pragma unroll
    for (int b = 0; b < kMB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

    // A fragment (32x32x16) of pixel block pb, slice h of a block: lane l
    // holds pixel 32 pb + (l & 31), channels 16 h + 8 (l >> 5) .. +7, by two
    // transposed reads of four channel rows each (16-lane group g covers
    // pixels 16 (g & 1) .. +15 and channel half g >> 1).
    const int grp = lane >> 4, jl = lane & 15;
    const int tr_off = (8 * (grp >> 1) + (jl >> 2)) * kPitch + 2 * (16 * (grp & 1) + 4 * (jl & 3));
    auto read_a = [&](const unsigned char *buf, int h, int pb) {
        const unsigned char *p = buf + tr_off + h * 16 * kPitch + 64 * pb;
        const u32x2 lo = lds_tr(p), hi2 = lds_tr(p + 4 * kPitch);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi2.x, hi2.y});
    };

    // Block b (unrolled: C_in <= 256 gives at most 8): write block b
    // (registers, slot b mod 2) to LDS buffer b mod 2 and request block b + 2
    // into the same registers; barrier; 2 x 7 MFMAs
    // with the fragment reads kDepth ahead.  The buffer written in block b
    // was last read in block b - 2, which every wave finished before the
    // barrier of block b - 1.
    bf16x8 fa[kDepth];
    auto run_block = [&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value, d = b % PD;
        unsigned char *buf = xs[b % 2];
        store_block(buf, xr_[d]);
        if constexpr (b + PD < NB) load_block(b + PD, xr_[d]);
        __syncthreads();
        u32x4 wcur[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int o = 2 * (2 * b + h) + hi;  // octet of k = 32 b + 16 h + 8 hi
            wcur[h] = o < OCT ? *(const u32x4 *)(wsm + (wrow * OCT + (o ^ (wrow & SW))) * 16) : u32x4{0u, 0u, 0u, 0u};
        }
        constexpr int kM = 2 * kMB;
        static_for<0, kDepth>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            fa[m] = read_a(buf, m / kMB, m % kMB);
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, kM>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int h = m / kMB, pb = m % kMB;
            const u32x4 wv = wcur[h];
            acc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m % kDepth], __builtin_bit_cast(bf16x8, wv), acc[pb],
                                                              0, 0, 0);
            if constexpr (m + kDepth < kM) fa[(m + kDepth) % kDepth] = read_a(buf, (m + kDepth) / kMB, (m + kDepth) % kMB);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    static_for<0, NB>([&](auto bc) { run_block(bc); });

    // Epilogue: BN + SiLU on the accumulators (lane: channel co; per block pb
    // and q, pixels 32 pb + 8 q + 4 hi .. +3), bf16, staged in LDS as the
    // wave's [32 channels][L pixels] tile over the weight tile (every wave is
    // past its last weight read after the barrier); each 32-pixel block is
    // stored as 16-byte pieces along its channel rows as soon as it is
    // staged.
    __syncthreads();
    unsigned char *const ot = wsm + wave * 32 * kEpiPitch;
    // With H*W and L multiples of 32 every such 64-byte piece is one whole
    // aligned segment of y (an image boundary inside the range falls between
    // blocks), and the stores take the streaming policy.
    const bool whole_segments = ((hw | L) & 31) == 0;
#pragma unroll
    for (int pb = 0; pb < kMB; ++pb) {
        if (32 * pb >= len) continue;  // uniform: blocks past a short range
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v0 = acc[pb][4 * q], v1 = acc[pb][4 * q + 1];
            const float v2 = acc[pb][4 * q + 2], v3 = acc[pb][4 * q + 3];
            u32x2 o;
            if (EPI == kFused) {
                o.x = pack_bf16x2(bn_silu(v0, sc, bi), bn_silu(v1, sc, bi));
                o.y = pack_bf16x2(bn_silu(v2, sc, bi), bn_silu(v3, sc, bi));
            } else {
                o.x = pack_bf16x2(v0, v1);
                o.y = pack_bf16x2(v2, v3);
            }
            *(u32x2 *)(ot + l32 * kEpiPitch + 2 * (32 * pb + 8 * q + 4 * hi)) = o;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        // The block's 32 channel rows x 4 pieces of 8 pixels: four
        // consecutive lanes write the block's 64 bytes of one channel row.
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = lane + 64 * i, r = t >> 2, col = 4 * pb + (t & 3);
            int n, p;
            pix(8 * col, n, p);
            const int c = ct * kTileCo + wave * 32 + r;
            const u32x4 v = *(const u32x4 *)(ot + r * kEpiPitch + 16 * col);
            const uint32_t off = (c < s.C_out && 8 * col < len) ? (uint32_t)((n * s.C_out + c) * hw + p) * 2u : kOOB;
            if (whole_segments) buf_store16_nt(yr, off, v);
            else buf_store16(yr, off, v);
        }
    }
}

// Pixels per range: the M pixels split evenly over one workgroup per CU,
// rounded up to a multiple of 8, at most 224 and at most one image.  When
// every CU would get at least 3/4 of a full range, full ranges are used
// instead (fewer, longer workgroups: the 1x1 layer at N=8, 256 -> 256,
// 80x80 runs 1.7% faster with 229 ranges of 224 pixels than with 256 of
// 200, measured).
int range_len(const Shape &s, int num_cu) {
    const int co_tiles = (s.C_out + kTileCo - 1) / kTileCo;
    const int per = (int)(((int64_t)s.M * co_tiles + num_cu - 1) / num_cu);
    int L = (per + 7) / 8 * 8;
    if (4 * L >= 3 * kMaxL) L = kMaxL;
    if (L > kMaxL) L = kMaxL;
    if (L > s.HW) L = s.HW;
    if (L < 8) L = 8;
    return L;
}

template <int KS, int EPI>
hipError_t launch_pw(const Shape &s, const void *x, const void *w, const float *scale, const float *bias, void *y,
                     hipStream_t st, int num_cu) {
    const int co_tiles = (s.C_out + kTileCo - 1) / kTileCo;
    const int L = range_len(s, num_cu);
    const int n_ranges = (s.M + L - 1) / L;
    const int items = n_ranges * co_tiles;
    hipLaunchKernelGGL((pointwise_bf16<KS, kPD, EPI>), dim3(items), dim3(kThreadsPw), 0, st, (const uint16_t *)x,
                       (const uint16_t *)w, scale, bias, (uint16_t *)y, s, L, n_ranges, co_tiles);
    return hipGetLastError();
}

}  // namespace

bool pointwise_supports(const Shape &s, int dtype) {
    return dtype == kDtypeBf16 && s.KH == 1 && s.KW == 1 && s.stride == 1 && s.pad == 0 && s.C_in % 8 == 0 &&
           s.C_in <= 256 && s.HW % 8 == 0 && (uint64_t)s.N * s.C_in * s.HW * 2 <= kMaxBufferBytes &&
           (uint64_t)s.N * s.C_out * s.HW * 2 <= kMaxBufferBytes;
}

bool pointwise_pointers_ok(const void *x, const void *w, const void *y) {
    return (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) == 0;
}

hipError_t launch_pointwise(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                            const float *bias, void *y, hipStream_t st, int num_cu) {
    const int ks = (s.C_in + 15) / 16;
#define CBS_PW(KS_)                                                                                 \
    if (ks <= KS_)                                                                                  \
        return epi == kFused ? launch_pw<KS_, kFused>(s, x, w, scale, bias, y, st, num_cu)          \
                             : launch_pw<KS_, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
    CBS_PW(4) CBS_PW(8) CBS_PW(16)
#undef CBS_PW
    return hipErrorInvalidValue;
}

}  // namespace cbs
