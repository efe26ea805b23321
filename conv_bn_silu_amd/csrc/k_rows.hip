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
//  * Workgroups of 4 waves, one per CU; wave w owns output channels
//    32w .. 32w+31 of the workgroup's 128-channel tile and all OW pixels of
//    the output row being computed (NB blocks of 32, v_mfma_f32_32x32x16_bf16).
//  * The G workgroups of a channel tile interleave over the N*OH output rows
//    (rank j takes rows j, j+G, ...): at any time the chip streams one
//    contiguous window of x and y, which keeps DRAM pages open.
//  * A unit is (output row, 16-channel chunk): its 48 input row segments
//    are loaded two units ahead into registers (16-byte loads of 8 columns,
//    split into even and odd columns with byte permutes), written to one of
//    three LDS sets during the unit before the one that reads it, and read
//    after the next barrier.  The copy tasks of a thread are spread over
//    that unit's steps, one after the matrix instructions of each step 1..8,
//    each followed by the load that reuses its registers, so the permutes
//    and LDS writes issue between matrix instructions (measured 1-3% faster
//    on the stride-2 layer at N=16, 64 -> 128, 320x320 than writing all of
//    them at the start of the unit).
//    The shifted odd array needs the column left of each segment: a wave's
//    load covers 63 consecutive segments in lanes 1..63 and repeats the one
//    before them in lane 0, so every lane takes that column from the lane
//    below it by a DPP wave shift (lane 0 only supplies it).
//  * The loop body is two output rows (all their chunks, unrolled), each
//    with its own set of accumulators: every iteration issues the same
//    memory operations in the same order, so the waits for each unit's data
//    count exactly the operations issued since and never drain the loads in
//    flight for the units ahead.
//  * Each wave keeps its weights (32 channels x C_in*9 k, 9 fragments of 16
//    bytes per lane and chunk) in registers for the whole kernel: a unit
//    issues no weight loads.
//  * Row pitch in LDS: 2*OW bytes, an odd multiple of 64 for OW = 32*NB
//    with NB odd (and padded to one otherwise), so the four rows a 16-lane
//    group reads fall in distinct quarters of the 64 banks.
//  * Epilogue: folded BN + SiLU, bf16, for a row while the next row is
//    computed into the other accumulator set, in ten pieces placed after the
//    matrix instructions of chosen steps, so that its arithmetic and stores
//    fill the gaps between them.  A lane holds 4-pixel groups of one channel
//    and its partner 32 lanes away the groups beside them; the two swap one
//    group each (ds_bpermute), so that each stores 16-byte pieces of 8
//    consecutive pixels (8-byte pieces of 4 when OW is not a multiple of 8).
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

constexpr int kRowsWaves = 4;
constexpr int kRowsThreads = 64 * kRowsWaves;
constexpr int kRowsTile = 32 * kRowsWaves;  // output channels per workgroup
constexpr int kChunk = 16;                  // input channels per unit
constexpr int kKRows = kChunk * 9;          // k rows per unit (144 = 9 MFMA steps of 16)
constexpr int kRowsPD = 2;                  // units of input in flight in registers
constexpr int kSets = 3;                    // LDS sets of k rows

template <int NB>
struct RowsGeo {
    static constexpr int OWMAX = 32 * NB;
    static constexpr int P = (NB % 2 == 1) ? 2 * OWMAX : 2 * OWMAX + 64;  // row pitch, odd multiple of 64
    static constexpr int SET = kKRows * P;                                // bytes per set
    // 16-byte tasks per unit: 3 input rows x 16 channels x (2*OWMAX)/8
    // segments, 63 new ones per wave-wide load
    static constexpr int TASKS = 3 * kChunk * (2 * OWMAX / 8);
    static constexpr int MAXT = ((TASKS + 62) / 63 + kRowsWaves - 1) / kRowsWaves;
};

// NCH: 16-channel chunks of C_in (C_in = 16 * NCH); W8: OW % 8 == 0.
template <int NB, int NCH, bool W8, int EPI>
__global__ __launch_bounds__(kRowsThreads, 1) void rows_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int co_tiles, int ranks_per_xcd,
    int n_ranks) {
    using G = RowsGeo<NB>;
    __shared__ __attribute__((aligned(16))) unsigned char sets[kSets * G::SET];
    // Target of the staging writes of idle lanes, so that the writes need no
    // branch and can be scheduled among the matrix instructions.
    __shared__ __attribute__((aligned(16))) unsigned char sink[2 * G::P + 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const int units = steps * nchunks;  // units from this index on (a padding row) load zeros, store nothing
    const int segs = s.W / 8;
    const int tasks = 3 * kChunk * segs;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.H * s.W * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)s.C_out * s.K * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);

    // Copy task q of this thread: segment t = 63 (4 q + wave) + lane - 1 of
    // the unit, i.e. input row kh of the unit, channel ci of the chunk,
    // 8-column segment seg.  Consecutive lanes hold consecutive segments;
    // lane 0 holds the segment before lane 1's and is only loaded.
    int tk_kh[G::MAXT], tk_lds[G::MAXT];
    uint32_t tk_goff[G::MAXT];
    bool tk_load[G::MAXT], tk_valid[G::MAXT], tk_first[G::MAXT];
#pragma unroll
    for (int q = 0; q < G::MAXT; ++q) {
        const int traw = 63 * (q * kRowsWaves + wave) + lane - 1;
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

    struct UnitPos {
        int n, oh, chunk;
    };
    auto unit_pos = [&](int u) {  // uniform
        const int t = u / nchunks, c = u - t * nchunks;
        const int row = j + t * n_ranks;
        const int n = row / s.OH;
        return UnitPos{n, row - n * s.OH, c};
    };

    // Copy task q of unit u: its 16-byte load (8 input columns), issued
    // against the unit's base offset in x.
    struct LoadBase {
        uint32_t base;
        int ih0;
        bool live;
    };
    auto load_base = [&](int u) {
        const UnitPos up = unit_pos(u);
        const int ih0 = 2 * up.oh - 1;  // first input row of the unit
        return LoadBase{(uint32_t)(((up.n * s.C_in + up.chunk * kChunk) * s.H + ih0) * s.W) * 2u, ih0, u < units};
    };
    auto load_task = [&](const LoadBase &lb, u32x4 &a, int q) {
        const int ih = lb.ih0 + tk_kh[q];
        const bool ok = lb.live && tk_load[q] && (uint32_t)ih < (uint32_t)s.H;
        a = buf_load16(xr, ok ? lb.base + tk_goff[q] : kOOB);
    };
    // Split task q's 8 input columns into the unit's three tap arrays (4
    // output pixels each) in LDS set `set`.
    auto write_task = [&](unsigned char *set, const u32x4 &v, int q) {
        const uint32_t e0 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
        const uint32_t e1 = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
        const uint32_t o0 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
        const uint32_t o1 = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
        // High half: column 8 seg - 1, the last odd column of the lane
        // below (wave_shr:1); none left of the row: zero padding.
        uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o1, 0x138, 0xf, 0xf, false);
        prev = tk_first[q] ? 0u : prev;
        unsigned char *dst = tk_valid[q] ? set + tk_lds[q] : sink;
        *(u32x2 *)(dst) = u32x2{__builtin_amdgcn_perm(o0, prev, 0x05040302u), __builtin_amdgcn_alignbit(o1, o0, 16)};
        *(u32x2 *)(dst + G::P) = u32x2{e0, e1};
        *(u32x2 *)(dst + 2 * G::P) = u32x2{o0, o1};
    };
    u32x4 ra[kRowsPD][G::MAXT];
    auto load_unit = [&](int u, u32x4 (&a)[G::MAXT]) {
        const LoadBase lb = load_base(u);
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) load_task(lb, a[q], q);
    };
    auto write_unit = [&](unsigned char *set, const u32x4 (&a)[G::MAXT]) {
#pragma unroll
        for (int q = 0; q < G::MAXT; ++q) write_task(set, a[q], q);
    };

    // Weights: lane holds output channel co_lane and, for chunk c and MFMA
    // step ks (0..8), k = c*144 + 16*ks + 8*(lane>>5) .. +7 (the OIHW row of
    // w restricted to the chunk's channels is contiguous).
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

    // A fragment geometry (32x32x16): lane l holds pixel l&31 of the block and
    // k = 16*ks + 8*(l>>5) .. +7.  16-lane group G = l>>4 covers pixels
    // 16*(G&1) .. +15 and k half G>>1; lane jj = l&15 of the group loads k-row
    // 16*ks + 8*(G>>1) + (jj>>2) (+4 for the second read) at pixels
    // 16*(G&1) + 4*(jj&3) .. +3.
    const int grp = lane >> 4, jl = lane & 15;
    const int tr_off = (8 * (grp >> 1) + (jl >> 2)) * G::P + 2 * (16 * (grp & 1) + 4 * (jl & 3));

    // Two accumulator sets: the two output rows of a loop iteration use one
    // each, and the first matrix instruction of a row starts from zero.
    // While a row is computed, the previous row's epilogue runs from the
    // other set in ten pieces placed among the matrix instructions.
    f32x16 accs[2][NB];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) accs[r][b][e] = 0.f;

    // Prologue: units 0..PD-1 in flight; unit 0 written to set 0.
    rows_for<0, kRowsPD>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        load_unit(d, ra[d]);
    });
    write_unit(sets, ra[0]);
    load_unit(kRowsPD, ra[0]);

    // Piece i of the epilogue of the rank's output row t, from accumulator
    // set pa (stores dropped for t < 0, before the first row, and for a
    // padding row t >= steps): pixel block i / 2, groups q = 2p, 2p+1 with
    // p = i % 2; lane holds channel co_lane, group q pixels
    // 32b + 8q + 4*(lane>>5) .. +3.  A lane and its partner 32 lanes away
    // swap one group each (ds_bpermute), so that each stores a 16-byte piece
    // of 8 consecutive pixels (8-byte pieces of 4 when OW is not a multiple
    // of 8).
    constexpr int kPieces = 2 * NB;
    auto epi_piece = [&](int t, const f32x16 (&pa)[NB], auto ic) {
        constexpr int i = decltype(ic)::value, b = i / 2, p = i % 2;
        const bool live = t >= 0 && t < steps;
        const UnitPos up = unit_pos((live ? t : 0) * nchunks);
        const uint32_t obase = (uint32_t)(((up.n * s.C_out + co_lane) * s.OH + up.oh) * s.OW) * 2u;
        const bool cok = co_lane < s.C_out && live;
        const int hl = lane >> 5;
        u32x2 g[2];
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * p + qq;
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = EPI == kFused ? bn_silu(pa[b][4 * q + r], sc, bi) : pa[b][4 * q + r];
            g[qq] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
        if constexpr (W8) {
            // The lower half-wave keeps group 2p and takes the partner's
            // (pixels 8(2p) + 4 .. +7); the upper keeps group 2p+1 and takes
            // the partner's (pixels 8(2p+1) .. +3).
            const int partner = 4 * (lane ^ 32);
            const u32x2 send = hl ? g[0] : g[1];
            const u32x2 recv{(uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)send.x),
                             (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)send.y)};
            const u32x4 v = hl ? u32x4{recv.x, recv.y, g[1].x, g[1].y} : u32x4{g[0].x, g[0].y, recv.x, recv.y};
            const int px = 32 * b + 8 * (2 * p + hl);
            buf_store16(yr, cok && px < s.OW ? obase + 2u * px : kOOB, v);
        } else {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int px = 32 * b + 8 * (2 * p + qq) + 4 * hl;
                buf_store8(yr, cok && px < s.OW ? obase + 2u * px : kOOB, g[qq]);
            }
        }
    };

    // Unit u (chunk ch of the iteration's row rc): barrier; then compute
    // unit u from set u%3 into accumulator set rc while writing unit u+1
    // into set (u+1)%3 and requesting unit u+1+PD, task by task between the
    // matrix instructions.  Set u%3 was written before this barrier; set
    // (u+1)%3 was last read in unit u-2, which every wave finished before
    // the barrier of unit u-1, and is complete before the barrier of unit
    // u+1 (the last task follows step 8).  After step ks of chunk ch come
    // the epilogue pieces i of the previous row (set 1 - rc) whose slot
    // floor(i * 9 * NCH / (2 NB)) is ch * 9 + ks: the row's ten pieces are
    // spread over its units' steps.
    auto run_unit = [&](int u, auto dc, auto chc, auto rcc) {
        constexpr int d = decltype(dc)::value;  // (u+1) % 2: register slot of unit u+1
        constexpr int ch = decltype(chc)::value, rc = decltype(rcc)::value;
        f32x16(&acc)[NB] = accs[rc];
        __syncthreads();
        unsigned char *const set_next = sets + ((u + 1) % kSets) * G::SET;
        const LoadBase lb_next = load_base(u + 1 + kRowsPD);
        const unsigned char *set = sets + (u % kSets) * G::SET;
        const u32x4(&wcurf)[9] = wres[ch];
        const int t_prev = u / nchunks - 1;
        // The fragments of step ks+1 are read while the NB matrix
        // instructions of step ks run (two fragment sets).
        bf16x8 af[2][NB];
        auto read_step = [&](int ks, bf16x8 (&a)[NB]) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const unsigned char *p = set + tr_off + ks * 16 * G::P + 64 * b;
                const u32x2 lo = rows_tr(p);
                const u32x2 hi = rows_tr(p + 4 * G::P);
                a[b] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
            }
        };
        read_step(0, af[0]);
        rows_for<0, 9>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            if constexpr (ks + 1 < 9) read_step(ks + 1, af[(ks + 1) & 1]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if constexpr (ch == 0 && ks == 0)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][b], __builtin_bit_cast(bf16x8, wcurf[0]),
                                                                     f32x16{}, 0, 0, 0);
                else
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[ks & 1][b], __builtin_bit_cast(bf16x8, wcurf[ks]), acc[b], 0, 0, 0);
            }
            rows_for<0, kPieces>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i * 9 * NCH / kPieces == ch * 9 + ks) epi_piece(t_prev, accs[1 - rc], ic);
            });
            // Copy task q of unit u+1 after the matrix instructions of step
            // 1 + q*8/MAXT, its register then reloaded for unit u+1+PD.
            rows_for<0, G::MAXT>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                if constexpr (1 + q * 8 / G::MAXT == ks) {
                    write_task(set_next, ra[d][q], q);
                    load_task(lb_next, ra[d][q], q);
                }
            });
        });
    };
    static_assert(kRowsPD == 2, "register slots alternate with unit parity");
    // Two output rows per iteration (the unit count 2 NCH is even, so the
    // register slots of the units repeat); a padding row past `steps`
    // computes on zeros and stores nothing.
    constexpr int UPI2 = 2 * NCH;
    const int iters2 = (steps + 1) / 2;
    for (int it = 0; it < iters2; ++it) {
        rows_for<0, UPI2>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            run_unit(it * UPI2 + c, std::integral_constant<int, (c + 1) % 2>{}, std::integral_constant<int, c % NCH>{},
                     std::integral_constant<int, c / NCH>{});
        });
    }
    // The last row computed (row 2*iters2 - 1, in set 1; a padding row if it
    // is past `steps`) is still pending.
    rows_for<0, kPieces>([&](auto ic) { epi_piece(2 * iters2 - 1, accs[1], ic); });
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
