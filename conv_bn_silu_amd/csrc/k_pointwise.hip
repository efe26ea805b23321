// k_pointwise.hip -- the 1x1 (stride 1, no padding) layer as a streaming GEMM.
//
// For a 1x1 convolution the implicit GEMM has no window: row m of the pixel
// operand is x[n][:][p] with m = n*H*W + p, so "read x once, write y once"
// (page "Fusing an Epilogue", section "The problem") means streaming x and y
// through the chip exactly once.  This kernel is built for that:
//
//  * Persistent workgroups, one per compute unit, of 8 waves (two per SIMD),
//    each with a tile of 256 output channels.  The pixels are cut into
//    chunks of CP and dealt round-robin: workgroup rank j computes chunks
//    j, j + G, j + 2G, ... (G ranks), so the whole chip streams through x
//    and y as one contiguous front (see the kernel for why that matters).
//  * XCD-aware placement: consecutive ranks run on one XCD, so chunks that
//    share cache lines, and x re-read by several channel tiles, meet in one
//    L2.
//  * The weight tile (256 channels x C_in) is fetched once per workgroup with
//    LDS DMA in coalesced pieces, then each wave keeps its 32 channels in
//    VGPRs for the whole kernel (the B operand of every MFMA, 16 bytes per
//    lane each).
//  * The products run on v_mfma_f32_32x32x16_bf16 (32 pixels x 32 channels x
//    16 k per instruction), the shape that sustains the matrix-core rate with
//    one wave per SIMD.
//  * x chunks are stored in LDS as channel records: per 32-channel block,
//    one 64-byte record per pixel, its four 16-byte octets XOR-swizzled with
//    bits 1..2 of the pixel index.  An MFMA A fragment -- eight consecutive
//    channels of one pixel per lane -- is then one ds_read_b128, and the 32
//    pixels x 2 octets that a wave reads at once hit distinct banks.  (On
//    gfx950 a transposed ds_read_b64_tr_b16 moves about a quarter of the
//    bytes per cycle of a plain 16-byte read, so the transposition is done
//    in registers while staging instead: a task loads 2 channels x 8 pixels,
//    16 bytes per channel, and writes the pair into 8 pixels' records.)
//  * Two chunks of x are in flight in registers while one is computed (four
//    measured no faster: the steady state is at the mixed read/write rate).
//  * The epilogue (folded BN, SiLU, bf16 rounding) runs on the accumulators;
//    each wave stages its 32-channel output tile in LDS and writes y in whole
//    128-byte rows, 16 bytes per lane.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

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

// Byte offset of octet `octet` (0..3) of the 64-byte record of pixel `px`
// within a record block: the octets are XOR-swizzled with bits 1..2 of the
// pixel so that 8 consecutive lanes reading one octet of 8 consecutive
// pixels, and the staging writes, spread over the banks.
__device__ __forceinline__ uint32_t rec_off(int px, int octet) {
    return (uint32_t)px * 64u + (((uint32_t)octet ^ ((uint32_t)px >> 1)) & 3u) * 16u;
}

constexpr int kWaves = 8;               // wave w owns output channels [32w, 32w+32) of the tile
constexpr int kThreadsPw = 64 * kWaves;
constexpr int kTileCo = 32 * kWaves;    // output channels per workgroup

// KS: 16-channel slices of C_in (C_in <= 16*KS); CP: pixels per chunk; PD:
// chunks in flight; EPI: fused epilogue or the bare convolution.
template <int KS, int CP, int PD, int EPI>
__global__ __launch_bounds__(kThreadsPw, 1) void pointwise_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int co_tiles, int ranks_per_xcd,
    int n_ranks) {
    constexpr int KP = KS * 16;                        // channels held in LDS (zero beyond C_in)
    constexpr int NKB = (KP + 31) / 32;                // 32-channel record blocks
    // Bytes per record block of a chunk, padded by one record so that the
    // blocks start in different banks (the staging writes of one instruction
    // cover several blocks).
    constexpr int KBB = CP * 64 + 64;
    constexpr int NPAIR = KP / 2;                      // channel pairs
    constexpr int NTASK = NPAIR * (CP / 8);            // staging tasks: 2 channels x 8 pixels
    constexpr int TPT = (NTASK + kThreadsPw - 1) / kThreadsPw;  // tasks per thread
    constexpr int MB = CP / 32;                        // 32-pixel blocks per chunk
    constexpr int OROW = CP + 8;                       // output staging: elements per channel row
    // One LDS area, used first for the workgroup's weight tile (kTileCo
    // channels x KP, loaded with LDS DMA) and then for the x chunks and the
    // output staging.
    constexpr int OCT = KP / 8;                        // 16-byte octets per weight row
    constexpr int W_BYTES = kTileCo * KP * 2;
    constexpr int XS_BYTES = 2 * NKB * KBB;
    constexpr int OS_BYTES = kWaves * 32 * OROW * 2;
    constexpr int LDS_BYTES = W_BYTES > XS_BYTES + OS_BYTES ? W_BYTES : XS_BYTES + OS_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    unsigned char(*const xs)[NKB * KBB] = (unsigned char(*)[NKB * KBB])lds;
    uint16_t(*const os)[32 * OROW] = (uint16_t(*)[32 * OROW])(lds + XS_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Work: the M pixels in chunks of CP, chunk c = j + t*n_ranks going to
    // rank j (its t-th chunk) of channel tile ct.  At any time the ranks
    // together read one contiguous stretch of every channel plane of x (and
    // write one of y), which keeps DRAM pages open; giving each workgroup a
    // run of its own spreads the accesses over every plane instead and
    // costs several microseconds of first-access latency.  XCD-aware: the
    // XCDs take blocks round-robin (XCD = block id % 8), and XCD x holds
    // ranks x*ranks_per_xcd .. +ranks_per_xcd-1 of every channel tile, so
    // neighbouring chunks (which share cache lines) meet in one L2.
    int j, ct;
    {
        const int b = (int)blockIdx.x;
        const int xcd = b & 7, slot = b >> 3;
        ct = slot % co_tiles;
        j = xcd * ranks_per_xcd + slot / co_tiles;
        if (slot / co_tiles >= ranks_per_xcd || j >= n_ranks) return;  // uniform
    }
    const int co_lane = ct * kTileCo + wave * 32 + (lane & 31);  // this lane's output channel
    const int n_total = (s.M + CP - 1) / CP;
    if (j >= n_total) return;  // uniform
    const int n_chunks = (n_total - j + n_ranks - 1) / n_ranks;  // chunks of this rank
    const int hw = s.HW;
    auto chunk_pos = [&](int c) {  // first pixel of this rank's chunk c (uniform)
        const int m = (j + c * n_ranks) * CP;
        const int n = m / hw;
        return PixPos{n, m - n * hw};
    };

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * hw * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * hw * 2u);

    u32x4 wf[KS];  // weights (B fragments), from the LDS weight tile
    float sc, bi, sn, bn;


    // Staging task t < NTASK (t = tid + q*threads): channel pair cp = t %
    // NPAIR (channels 2cp, 2cp+1), 8-pixel piece t / NPAIR; two 16-byte
    // loads, and per pixel one 4-byte LDS write of the pair into the pixel's
    // record.  A piece outside the range, a channel past C_in, or a chunk past
    // the last, gets an out-of-range offset: the load returns zeros and costs
    // no memory traffic.
    auto load_chunk = [&](int c, u32x4 (&r)[TPT][2]) {
        const PixPos c0 = chunk_pos(c);
        const int mc = (j + c * n_ranks) * CP;
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
            const int t = tid + q * kThreadsPw;
            const int cp = t % NPAIR, piece = t / NPAIR;
            const PixPos pp = advance(c0, 8 * piece, hw);
            const bool ok = t < NTASK && c < n_chunks && mc + 8 * piece < s.M && 2 * cp < s.C_in;
            const uint32_t off0 = (uint32_t)((pp.n * s.C_in + 2 * cp) * hw + pp.p) * 2u;
            r[q][0] = buf_load16(xr, ok ? off0 : kOOB);
            r[q][1] = buf_load16(xr, ok ? off0 + (uint32_t)hw * 2u : kOOB);
        }
    };
    auto store_chunk = [&](int buf, const u32x4 (&r)[TPT][2]) {
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
            const int t = tid + q * kThreadsPw;
            if (TPT * kThreadsPw != NTASK && t >= NTASK) continue;
            const int cp = t % NPAIR, piece = t / NPAIR;
            unsigned char *blk = &xs[buf][(cp >> 4) * KBB] + (cp & 3) * 4;  // block, word in octet
            const int oct = (cp >> 2) & 3;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t lo = r[q][0][p >> 1], hi = r[q][1][p >> 1];
                const uint32_t v = (p & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                                           : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                *(uint32_t *)(blk + rec_off(8 * piece + p, oct)) = v;
            }
        }
    };

    // A fragment of 16-channel slice ks for 32-pixel block i (32x32x16: lane
    // l holds pixel l&31, channels 16*ks + 8*(l>>5) .. +7).
    uint16_t *const ow = os[wave];
    auto read_a = [&](int buf, int ks, int i) {
        return *(const bf16x8 *)(&xs[buf][(ks >> 1) * KBB + rec_off(32 * i + (lane & 31), 2 * (ks & 1) + (lane >> 5))]);
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
        const PixPos c0 = chunk_pos(live ? c : 0);
        const int mc = (j + (live ? c : 0) * n_ranks) * CP;
        constexpr int PIECES = CP / 8;          // 16-byte pieces per channel row
        constexpr int ROWS_PER = 64 / PIECES;   // rows covered by one wave-wide pass
#pragma unroll
        for (int k = 0; k < 32 / ROWS_PER; ++k) {
            const int r = k * ROWS_PER + lane / PIECES, piece = lane % PIECES;
            const u32x4 v = *(const u32x4 *)&ow[r * OROW + 8 * piece];
            const PixPos pp = advance(c0, 8 * piece, hw);
            const int co = ct * kTileCo + wave * 32 + r;
            const bool ok = live && mc + 8 * piece < s.M && co < s.C_out;
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
    // Weight tile first, with LDS DMA: rows co0 .. co0+255 of w, KP channels
    // each (zeros past C_out or C_in), 16-byte octet o of row r stored in
    // slot r*OCT + (o ^ (r & SW)): 16 lanes reading one octet of 16
    // consecutive rows hit 16 distinct bank groups, and each DMA instruction
    // still fetches contiguous pieces of a few rows.  Lane i of a DMA
    // instruction writes slot base + i, so the slot decides what it fetches.
    constexpr int SW = (OCT < 16 ? OCT : 16) - 1;
    {
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)s.C_out * s.C_in * 2u);
        const int co0 = ct * kTileCo;
#pragma unroll
        for (int j = 0; j < kTileCo * OCT / kThreadsPw; ++j) {
            const int slot = j * kThreadsPw + tid;
            const int r = slot / OCT, o = (slot % OCT) ^ (r & SW);
            const int co = co0 + r, k = 8 * o;
            const uint32_t off = (co < s.C_out && k < s.C_in) ? (uint32_t)(co * s.C_in + k) * 2u : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void *)(lds + (j * kThreadsPw + wave * 64) * 16), 16, off, 0, 0,
                0);
        }
    }
    u32x4 r[PD][TPT][2];
#pragma unroll
    for (int d = 0; d < PD; ++d) load_chunk(d, r[d]);

    // The epilogue constants are folded: v = acc*sc + bi, -v*log2(e) =
    // acc*sn + bn.
    sc = co_lane < s.C_out ? scale[co_lane] : 0.f;
    bi = co_lane < s.C_out ? bias[co_lane] : 0.f;
    sn = sc * -1.4426950408889634f;
    bn = bi * -1.4426950408889634f;

    // Weights into registers (B operand of the 32x32x16 MFMA): lane holds
    // channel co_lane and k = 16*ks + 8*(lane>>5) .. +7.  Octets past C_in
    // are forced to zero whatever the LDS holds.
    __builtin_amdgcn_s_waitcnt(0);  // the DMA above (and the first x chunks) have landed
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int rrow = wave * 32 + (lane & 31), o = 2 * ks + (lane >> 5);
        const u32x4 v = *(const u32x4 *)(lds + (rrow * OCT + (o ^ (rrow & SW))) * 16);
        wf[ks] = 8 * o < s.C_in ? v : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();  // the weight tile's LDS is reused for x from here on

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
    // One workgroup per compute unit in total, split over the channel tiles.
    const int n_total = (s.M + CP - 1) / CP;
    int n_ranks = (num_cu + co_tiles - 1) / co_tiles;
    if (n_ranks > n_total) n_ranks = n_total;
    const int ranks_per_xcd = (n_ranks + 7) / 8;
    const int blocks = ranks_per_xcd * 8 * co_tiles;
    hipLaunchKernelGGL((pointwise_bf16<KS, CP, PD, EPI>), dim3(blocks), dim3(kThreadsPw), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, co_tiles,
                       ranks_per_xcd, n_ranks);
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
        return epi == kFused ? launch_pw<KS_, 32, 2, kFused>(s, x, w, scale, bias, y, st, num_cu) \
                             : launch_pw<KS_, 32, 2, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
    CBS_PW(4) CBS_PW(8) CBS_PW(16)
#undef CBS_PW
    return hipErrorInvalidValue;
}

}  // namespace cbs
