// k_rows.hip -- 3x3, stride-2, padding-1 layers with a moderate channel
// count (C_in a multiple of 16, up to 64): the downsampling convolutions of
// a detector backbone.  Bound by streaming x in and y out.
//
// The GEMM view is the one of "Fusing an Epilogue" (section "Three kernels
// for one operation"), with the reduction k = (ci, kh, kw) in the OIHW order
// of w.  The A operand comes from LDS by transposed reads
// (ds_read_b64_tr_b16), which need the four pixels a lane loads to be
// adjacent and 8-byte aligned in LDS; with stride 2 the pixels of one tap
// are every other input column, so each input row is stored as three
// "horizontal im2col" arrays, one per tap column:
//     A_kw[ow] = x[ih][2*ow + kw - 1]   (zero outside the row),
// i.e. the odd columns shifted by one (kw = 0), the even columns (kw = 1)
// and the odd columns (kw = 2).  Array (ci, kh, kw) is row k of a
// [k][pixel] matrix, so a 16-k step of the MFMA reads 16 consecutive rows.
//
// Roles.  One workgroup of 8 waves per CU, two per SIMD: four consumers and
// four producers.  A consumer holds, for the whole kernel, the weights of 32
// output channels (9 fragments of 16 bytes per lane and chunk) and the
// accumulators of one output row (NB blocks of 32 pixels,
// v_mfma_f32_32x32x16_bf16); it only reads LDS and runs the matrix
// instructions and the epilogue arithmetic.  A producer only moves data:
// x from HBM into the LDS arrays, and finished rows of y from LDS to HBM.
// With the two roles in different waves of one SIMD, the matrix pipe is fed
// while the producer on the same SIMD waits for its loads, which one wave
// doing both (the register file then holds the weights, two accumulator
// sets and the loads in flight) cannot do.
//  * The G workgroups of a channel tile interleave over the N*OH output rows
//    (rank j takes rows j, j+G, ...): at any time the chip streams one
//    contiguous window of x and y, which keeps DRAM pages open.
//  * A unit is (output row, 16-channel chunk): its 48 input row segments.
//    The producers load them PD units ahead into registers (16-byte loads
//    of 8 columns, split into even and odd columns with byte permutes) and
//    write unit u+1 into one of two LDS sets while the consumers compute
//    unit u from the other; one barrier per unit.  The shifted odd array
//    needs the column left of each segment: a wave's load covers 63
//    consecutive segments in lanes 1..63 and repeats the one before them in
//    lane 0, so every lane takes that column from the lane below it by a DPP
//    wave shift (lane 0 only supplies it).
//  * After a row's last unit the consumers apply the folded BN + SiLU and
//    write the row, as bf16, into an LDS staging area ([channel][pixel],
//    pitch 2*OWMAX + 16 bytes); during the next row's units the producers
//    store it to y in 16-byte pieces, four consecutive lanes per 64-byte
//    segment of a channel row, with the non-temporal policy when OW is a
//    multiple of 32 (8-byte pieces when OW is not a multiple of 8).  A
//    second barrier per row separates those stores from the next row's
//    staging writes.
//  * Row pitch of the k arrays in LDS: 2*OW bytes, an odd multiple of 64
//    for OW = 32*NB with NB odd (and padded to one otherwise), so the four
//    rows a 16-lane group reads fall in distinct quarters of the 64 banks.
//  * Accumulation order per output: chunk by chunk, and within a chunk the
//    nine 16-k steps in order, the same for every shape.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 rows_tr(const unsigned char *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

template <int B, int E, typename F>
__device__ __forceinline__ void rows_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        rows_for<B + 1, E>(f);
    }
}

constexpr int kRowsWaves = 4;                      // consumer waves, and producer waves
constexpr int kRowsThreads = 2 * 64 * kRowsWaves;  // one consumer and one producer wave per SIMD
constexpr int kRowsTile = 32 * kRowsWaves;         // output channels per workgroup
constexpr int kChunk = 16;                         // input channels per unit
constexpr int kKRows = kChunk * 9;                 // k rows per unit (144 = 9 MFMA steps of 16)
constexpr int kRowsPD = 4;                         // units of input in flight in producer registers
constexpr int kSets = 2;                           // LDS sets of k rows
constexpr int kAhead = kSets - 1;                  // units written ahead of the one being computed
constexpr int kRing = 2;                           // A fragments in registers ahead of their MFMA
static_assert(kRowsPD >= kAhead, "the prologue writes kAhead units from the first slots");

template <int NB>
struct RowsGeo {
    static constexpr int OWMAX = 32 * NB;
    static constexpr int P = (NB % 2 == 1) ? 2 * OWMAX : 2 * OWMAX + 64;  // row pitch, odd multiple of 64
    static constexpr int SET = kKRows * P;                                // bytes per set
    // 16-byte copy tasks per unit: 3 input rows x 16 channels x (2*OWMAX)/8
    // segments, 63 new ones per wave-wide load, over the producer waves
    static constexpr int TASKS = 3 * kChunk * (2 * OWMAX / 8);
    static constexpr int MAXT = ((TASKS + 62) / 63 + kRowsWaves - 1) / kRowsWaves;
    static constexpr int YP = 2 * OWMAX + 16;                             // y staging pitch (bytes per channel)
    static constexpr int YSTAGE = kRowsTile * YP;
};

template <int NB, int NCH, bool W8, int EPI>
__global__ __launch_bounds__(kRowsThreads, 1) void rows_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int co_tiles, int ranks_per_xcd,
    int n_ranks) {
    using G = RowsGeo<NB>;
    __shared__ __attribute__((aligned(16))) unsigned char sets[kSets * G::SET];
    __shared__ __attribute__((aligned(16))) unsigned char ystage[G::YSTAGE];
    // Target of the staging writes of idle producer lanes, so that the writes
    // need no branch.
    __shared__ __attribute__((aligned(16))) unsigned char sink[2 * G::P + 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int j, ct;
    {
        const int b = (int)blockIdx.x;
        const int xcd = b & 7, slot = b >> 3;
        ct = slot % co_tiles;
        j = xcd * ranks_per_xcd + slot / co_tiles;
        if (slot / co_tiles >= ranks_per_xcd || j >= n_ranks) return;  // uniform
    }
    const int rows_total = s.N * s.OH;
    if (j >= rows_total) return;  // uniform
    const int steps = (rows_total - j + n_ranks - 1) / n_ranks;  // output rows of this rank
    constexpr int nchunks = NCH;
    const int units = steps * nchunks;

    struct UnitPos {
        int n, oh, chunk;
    };
    auto unit_pos = [&](int u) __attribute__((always_inline)) {  // uniform
        const int t = u / nchunks, c = u - t * nchunks;
        const int row = j + t * n_ranks;
        const int n = row / s.OH;
        return UnitPos{n, row - n * s.OH, c};
    };

    if (wave >= kRowsWaves) {
        // Producer: unit u+1 into set (u+1)%2 after the barrier of unit u
        // (that set was last read in unit u-1), then unit u+1+PD requested
        // into the freed registers, then a share of the previous row's y.
        // Units in flight: a multiple of NCH, so that the unrolled loop knows
        // each unit's chunk and register slot; two where the 8-byte output
        // pieces of the widest rows leave fewer registers (the time does not
        // depend on it between one and six units).
        constexpr int PD = NCH == 3 ? 3 : (NB == 5 && !W8 && NCH <= 2) ? 2 : kRowsPD;
        const int pw = wave - kRowsWaves;
        const int ptid = tid - 64 * kRowsWaves;
        const int segs = s.W / 8;
        const int tasks = 3 * kChunk * segs;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.H * s.W * 2u);
        const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);
        // Copy task q of this lane: segment t = 63 (4 q + pw) + lane - 1 of
        // the unit, i.e. input row kh of the unit, channel ci of the chunk,
        // 8-column segment seg.  Consecutive lanes hold consecutive segments;
        // lane 0 holds the segment before lane 1's and is only loaded.
        int tk_kh[G::MAXT], tk_lds[G::MAXT];
        uint32_t tk_goff[G::MAXT];
        bool tk_load[G::MAXT], tk_valid[G::MAXT], tk_first[G::MAXT];
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) {
            const int traw = 63 * (q * kRowsWaves + pw) + lane - 1;
            const int t = traw < 0 ? 0 : traw;
            const int kh = t / (kChunk * segs), rem = t - kh * (kChunk * segs);
            const int ci = rem / segs, seg = rem - ci * segs;
            tk_load[q] = traw >= 0 && t < tasks;
            tk_valid[q] = lane > 0 && t < tasks;
            tk_first[q] = seg == 0;
            tk_kh[q] = kh;
            tk_goff[q] = (uint32_t)((ci * s.H + kh) * s.W + 8 * seg) * 2u;
            tk_lds[q] = (ci * 9 + kh * 3) * G::P + 8 * seg;
        }
        struct LoadBase {
            uint32_t base;
            int ih0;
            bool live;
        };
        auto load_base = [&](int u) __attribute__((always_inline)) {
            const UnitPos up = unit_pos(u);
            const int ih0 = 2 * up.oh - 1;
            return LoadBase{(uint32_t)(((up.n * s.C_in + up.chunk * kChunk) * s.H + ih0) * s.W) * 2u, ih0,
                            u < units};
        };
        auto load_task = [&](const LoadBase &lb, u32x4 &a, int q) __attribute__((always_inline)) {
            const int ih = lb.ih0 + tk_kh[q];
            const bool ok = lb.live && tk_load[q] && (uint32_t)ih < (uint32_t)s.H;
            a = buf_load16(xr, ok ? lb.base + tk_goff[q] : kOOB);
        };
        auto write_task = [&](unsigned char *set, const u32x4 &v, int q) __attribute__((always_inline)) {
            const uint32_t e0 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
            const uint32_t e1 = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
            const uint32_t o0 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
            const uint32_t o1 = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
            uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o1, 0x138, 0xf, 0xf, false);
            prev = tk_first[q] ? 0u : prev;
            unsigned char *dst = tk_valid[q] ? set + tk_lds[q] : sink;
            *(u32x2 *)(dst) = u32x2{__builtin_amdgcn_perm(o0, prev, 0x05040302u), __builtin_amdgcn_alignbit(o1, o0, 16)};
            *(u32x2 *)(dst + G::P) = u32x2{e0, e1};
            *(u32x2 *)(dst + 2 * G::P) = u32x2{o0, o1};
        };
        // Output row t from the staging area to y: pieces k = part (mod NCH)
        // (part = NCH: all of them), piece p = k * 256 + ptid covering
        // channel p / ppr of the tile, pixels (p % ppr) * PX .. +PX-1, so that
        // consecutive lanes store consecutive pieces of a channel row.
        constexpr int PX = W8 ? 8 : 4;
        constexpr int KMAX = (kRowsTile * (G::OWMAX / PX) + 255) / 256;
        const int ppr = s.OW / PX;
        const int npieces = kRowsTile * ppr;
        const bool whole = (s.OW & 31) == 0;
        // A piece's place does not depend on the row: its staging offset and
        // its offset in y from the row's first element are computed once
        // (the division by ppr would otherwise cost the producers some thirty
        // vector instructions per piece, and their instructions are on the
        // critical path).
        int pk_src[KMAX];
        uint32_t pk_y[KMAX];
        bool pk_ok[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int p = k * 256 + ptid;
            const int col = p / ppr, pc = p - col * ppr;
            const int cog = ct * kRowsTile + col;
            pk_ok[k] = p < npieces && cog < s.C_out;
            pk_src[k] = (pk_ok[k] ? col : 0) * G::YP + pc * (2 * PX);
            pk_y[k] = pk_ok[k] ? (uint32_t)(cog * s.OHW + pc * PX) * 2u : 0u;
        }
        auto store_y = [&](int t, auto partc) __attribute__((always_inline)) {
            constexpr int part = decltype(partc)::value;
            const UnitPos up = unit_pos(t * nchunks);
            const uint32_t rowbase = (uint32_t)((up.n * s.C_out * s.OH + up.oh) * s.OW) * 2u;
            rows_for<0, KMAX>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (part == NCH || k % NCH == part) {
                const unsigned char *src = ystage + pk_src[k];
                const uint32_t off = pk_ok[k] ? rowbase + pk_y[k] : kOOB;
                if constexpr (W8) {
                    const u32x4 v = *(const u32x4 *)src;
                    if (whole) buf_store16_nt(yr, off, v);
                    else buf_store16(yr, off, v);
                } else {
                    buf_store8(yr, off, *(const u32x2 *)src);
                }
                }
            });
        };
        u32x4 ra[PD][G::MAXT];
        rows_for<0, PD>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            const LoadBase lb = load_base(d);
            rows_for<0, G::MAXT>([&](auto qc) { load_task(lb, ra[d][decltype(qc)::value], decltype(qc)::value); });
        });
        rows_for<0, kAhead>([&](auto ac) {
            constexpr int a = decltype(ac)::value;
            const LoadBase lb = load_base(PD + a);
            rows_for<0, G::MAXT>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                write_task(sets + a * G::SET, ra[a][q], q);
                load_task(lb, ra[a][q], q);
            });
        });
        static_assert(PD % NCH == 0, "a unit's chunk is known at compile time");
        auto pstep = [&](int u, auto cc) __attribute__((always_inline)) {
            constexpr int slot = (decltype(cc)::value + kAhead) % PD;
            constexpr int part = decltype(cc)::value % NCH;
            __syncthreads();
            const int v = u + kAhead;
            unsigned char *const set = sets + (v % kSets) * G::SET;
            const LoadBase lb = load_base(v + PD);
            rows_for<0, G::MAXT>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                write_task(set, ra[slot][q], q);
                load_task(lb, ra[slot][q], q);
            });
            const int t = u / nchunks;
            if (t > 0) store_y(t - 1, std::integral_constant<int, part>{});
            if constexpr (part == NCH - 1) __syncthreads();  // the row's y staging barrier
        };
        int u = 0;
        for (; u + PD <= units; u += PD)
            rows_for<0, PD>([&](auto cc) { pstep(u + decltype(cc)::value, cc); });
        rows_for<0, PD>([&](auto cc) {
            if (u + decltype(cc)::value < units) pstep(u + decltype(cc)::value, cc);
        });
        __syncthreads();  // the last row is staged
        store_y(steps - 1, std::integral_constant<int, NCH>{});
        return;
    }

    // Consumer: barrier, unit u from set u%2; after a row's last unit, the
    // row barrier (the producers are done with the staging area), then the
    // epilogue into it.
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)s.C_out * s.K * 2u);
    const int co_lane = ct * kRowsTile + wave * 32 + (lane & 31);
    u32x4 wres[NCH][9];
    {
        const bool ok = co_lane < s.C_out;
        const uint32_t base = (uint32_t)(co_lane * s.K + 8 * (lane >> 5)) * 2u;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int ks = 0; ks < 9; ++ks) wres[c][ks] = buf_load16(wr, ok ? base + 2u * (c * kKRows + 16 * ks) : kOOB);
    }
    const float sc = co_lane < s.C_out ? scale[co_lane] : 0.f;
    const float bi = co_lane < s.C_out ? bias[co_lane] : 0.f;
    const int grp = lane >> 4, jl = lane & 15;
    const int tr_off = (8 * (grp >> 1) + (jl >> 2)) * G::P + 2 * (16 * (grp & 1) + 4 * (jl & 3));
    // Staging of a row's results: lane holds channel wave*32 + (lane&31) and,
    // per block b and group q, pixels 32b + 8q + 4*(lane>>5) .. +3.
    unsigned char *const ydst = ystage + (wave * 32 + (lane & 31)) * G::YP + 8 * (lane >> 5);

    f32x16 acc[NB];
    constexpr int NI = 9 * NB;
    for (int t = 0; t < steps; ++t) {
        rows_for<0, NCH>([&](auto chc) {
            constexpr int ch = decltype(chc)::value;
            __syncthreads();
            const int u = t * nchunks + ch;
            const unsigned char *set = sets + (u % kSets) * G::SET;
            bf16x8 fr[kRing];
            auto rd = [&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value, ks = i / NB, b = i % NB;
                const unsigned char *p = set + tr_off + ks * 16 * G::P + 64 * b;
                const u32x2 lo = rows_tr(p);
                const u32x2 hi = rows_tr(p + 4 * G::P);
                fr[i % kRing] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
            };
            rows_for<0, kRing - 1>([&](auto ic) { rd(ic); });
            rows_for<0, NI>([&](auto ic) {
                constexpr int i = decltype(ic)::value, ks = i / NB, b = i % NB;
                if constexpr (i + kRing - 1 < NI) rd(std::integral_constant<int, i + kRing - 1>{});
                if constexpr (ch == 0 && ks == 0)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % kRing],
                                                                     __builtin_bit_cast(bf16x8, wres[ch][ks]),
                                                                     f32x16{}, 0, 0, 0);
                else
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fr[i % kRing], __builtin_bit_cast(bf16x8, wres[ch][ks]), acc[b], 0, 0, 0);
            });
        });
        __syncthreads();  // the producers have stored the previous row from the staging area
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = acc[b][4 * q + r];
                if constexpr (EPI == kFused) {
                    // bn_silu on four values as four interleaved chains (the
                    // same operations; the scheduling barriers keep the
                    // compiler, short of registers here, from running them
                    // one after another, where each waits for its
                    // transcendentals: 84.7 -> 83.6 us on the stride-2 layer
                    // at N=16, 64 -> 128, 320x320, same bits).
                    float e[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = __builtin_fmaf(o[r], sc, bi);
#pragma unroll
                    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(o[r] * -1.4426950408889634f);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_rcpf(1.0f + e[r]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = o[r] * e[r];
                }
                *(u32x2 *)(ydst + 2 * (32 * b + 8 * q)) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
    }
    __syncthreads();  // the last row is staged
}

template <int NB, int NCH, bool W8, int EPI>
hipError_t launch_rows_t(const Shape &s, const void *x, const void *w, const float *scale, const float *bias,
                         void *y, hipStream_t st, int num_cu) {
    const int co_tiles = (s.C_out + kRowsTile - 1) / kRowsTile;
    const int rows_total = s.N * s.OH;
    int n_ranks = (num_cu + co_tiles - 1) / co_tiles;
    if (n_ranks > rows_total) n_ranks = rows_total;
    const int ranks_per_xcd = (n_ranks + 7) / 8;
    hipLaunchKernelGGL((rows_bf16<NB, NCH, W8, EPI>), dim3(ranks_per_xcd * 8 * co_tiles), dim3(kRowsThreads), 0, st,
                       (const uint16_t *)x, (const uint16_t *)w, scale, bias, (uint16_t *)y, s, co_tiles,
                       ranks_per_xcd, n_ranks);
    return hipGetLastError();
}

}  // namespace

bool rows_supports(const Shape &s, int dtype) {
    return dtype == kDtypeBf16 && s.KH == 3 && s.KW == 3 && s.stride == 2 && s.pad == 1 && s.C_in % kChunk == 0 &&
           s.C_in <= 64 && s.W % 8 == 0 && s.OW == s.W / 2 && s.OW % 4 == 0 && s.OW <= RowsGeo<5>::OWMAX &&
           (uint64_t)s.N * s.C_in * s.H * s.W * 2 <= kMaxBufferBytes &&
           (uint64_t)s.N * s.C_out * s.OHW * 2 <= kMaxBufferBytes;
}

bool rows_pointers_ok(const void *x, const void *w, const void *y) {
    return (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) == 0;
}

hipError_t launch_rows(const Shape &s, int epi, const void *x, const void *w, const float *scale, const float *bias,
                       void *y, hipStream_t st, int num_cu) {
#define CBS_ROWS3(NB_, NCH_, W8_)                                                                          \
    return epi == kFused ? launch_rows_t<NB_, NCH_, W8_, kFused>(s, x, w, scale, bias, y, st, num_cu)      \
                         : launch_rows_t<NB_, NCH_, W8_, kConvOnly>(s, x, w, scale, bias, y, st, num_cu);
#define CBS_ROWS2(NB_, NCH_)                                                                               \
    if (s.C_in == kChunk * NCH_) {                                                                         \
        if (s.OW % 8 == 0) CBS_ROWS3(NB_, NCH_, true)                                                      \
        CBS_ROWS3(NB_, NCH_, false)                                                                        \
    }
#define CBS_ROWS(NB_)                                                                                  \
    if (s.OW <= RowsGeo<NB_>::OWMAX) {                                                                 \
        CBS_ROWS2(NB_, 1) CBS_ROWS2(NB_, 2) CBS_ROWS2(NB_, 3) CBS_ROWS2(NB_, 4)                        \
        return hipErrorInvalidValue;                                                                   \
    }
    CBS_ROWS(1) CBS_ROWS(3) CBS_ROWS(5)
#undef CBS_ROWS
#undef CBS_ROWS2
#undef CBS_ROWS3
    return hipErrorInvalidValue;
}

}  // namespace cbs
