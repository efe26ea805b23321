// k_window32.hip -- implicit-GEMM 3x3 convolution on v_mfma_f32_32x32x16_bf16
// for the compute-bound layers (many channels, small images): the input
// window of a tile is staged in LDS once per 32-channel block and reused by
// all nine kernel taps, as in the 16x16 window kernel, but each wave holds a
// column of 7 32x32 accumulators so that every weight fragment read from LDS
// feeds 7 matrix instructions ("Fusing an Epilogue", section "Three kernels
// for one operation": the GEMM kernel has the best arithmetic intensity).
//
// Workgroup: 8 waves (two per SIMD, so that one wave's staging and waits
// hide behind the other's matrix work) as 2 (pixels) x 4 (channels); tile =
// TH x TW output pixels of one image x 128 output channels; wave (wm, wn)
// owns pixel blocks wm*MB .. wm*MB+MB-1 (32 pixels each, pixel p of the tile
// = row p / TW, column p mod TW) and output channels 32*wn .. +31.
//
// Reduction order: channel block (32 channels), then groups of three taps,
// then the tap, then two 16-channel halves.  LDS holds two window buffers
// (this channel block and the next) and two weight buffers (this tap group
// and the next); one barrier per tap group.  A record holds 32 channels of
// one input position (window) or one output channel (weights) in 64 bytes,
// padded to 80: with 5 16-byte slots per record, 16 lanes reading one slot of
// 16 consecutive records hit 16 distinct bank groups of gfx950's 64-bank LDS,
// and a fragment -- 8 consecutive channels of one pixel or one output
// channel per lane -- is one ds_read_b128 whose per-tap part of the address
// is a uniform offset.  The window's row pitch is chosen so that this holds
// across the row wraps of the tile too.
//
// Staging is through registers and runs well ahead of use: the next tap
// group's weights (3 x 16 bytes per thread) are requested at the start of a
// group and written at its end, and the next channel block's whole window
// (one or two parts of 512 tasks, each task 8 channels x VEC columns,
// transposed with byte permutes) is requested at the start of a block and
// written at its end.  Within a group the fragment reads run a fixed
// distance ahead of the matrix instructions.  The nine taps are unrolled with
// the stride fixed at compile time, and blocks advance by counters, so that
// the loop does no integer division: the scalar unit, shared by both waves
// of a SIMD, would otherwise issue more instructions per tap than the matrix
// core runs.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {

namespace {

constexpr int kThreads32 = 512;
constexpr int kBN32 = 128;            // output channels per tile
constexpr int kCK32 = 32;             // input channels per block
constexpr int kRec = 80;              // bytes per record (64 data + 16 padding)
constexpr int kFpBytes32 = 41 * 1024; // one window buffer
constexpr int kWTB = kBN32 * kRec;    // one tap's weights: 128 records
constexpr int kGT = 3;                // taps per weight group (one barrier each)
constexpr int kDepth = 4;             // fragment reads in flight ahead of the matrix instructions
// Window staging parts of 512 tasks: one for 16-byte loads, two for 8-byte
// loads (narrow images), which is what the register budget of two waves per
// SIMD allows.
constexpr int parts_for(int vec) { return vec == 8 ? 1 : 2; }

// Calls f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Half h of lo_word in the low half, half h of hi_word in the high half (one
// byte permute).
__device__ __forceinline__ uint32_t pair16(uint32_t lo_word, uint32_t hi_word, int h) {
    return __builtin_amdgcn_perm(hi_word, lo_word, h == 0 ? 0x05040100u : 0x07060302u);
}

template <int VEC> struct XV32;
template <> struct XV32<8> {
    typedef u32x4 T;
    __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) { return buf_load16(r, off); }
};
template <> struct XV32<4> {
    typedef u32x2 T;
    __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) { return buf_load8(r, off); }
};

// MB: 32-pixel blocks per wave; VEC: input columns per staging load (8 or
// 4); S: stride (1 or 2).
template <int MB, int VEC, int S, int EPI>
__global__ __launch_bounds__(kThreads32, 1) void window32_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, WinGeo g) {
    __shared__ __attribute__((aligned(16))) unsigned char fps[2][kFpBytes32];
    __shared__ __attribute__((aligned(16))) unsigned char wbs[2][kGT * kWTB];
    __shared__ __attribute__((aligned(16))) unsigned char sink[64 * 16];  // target of masked-off stores
    typedef typename XV32<VEC>::T XT;
    constexpr int kT = 9;  // taps
    constexpr int kParts = parts_for(VEC);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, hi = lane >> 5;

    // XCD-aware placement: the XCDs take workgroups round-robin (XCD =
    // block id mod 8); rank the workgroups so that each XCD runs one
    // contiguous range of tiles, which puts the 128-channel tiles of one
    // image (consecutive tile indices) on one XCD, where they share its L2
    // for the input window instead of each fetching it from memory.
    const int xcd = (int)blockIdx.x & 7, q8 = g.n_wg >> 3, r8 = g.n_wg & 7;
    const int rank = xcd * q8 + min(xcd, r8) + ((int)blockIdx.x >> 3);
    const int t_begin = rank * g.tiles_per_wg;
    const int t_end = min(t_begin + g.tiles_per_wg, g.n_tiles);
    if (t_begin >= t_end) return;  // uniform
    const int n_steps = (t_end - t_begin) * g.n_chunks;  // (tile, channel block) pairs

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.HW * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.C_out * g.n_chunks * kT * 64u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);

    // A block: one 32-channel slice of one tile.
    struct Blk {
        int tile, n, oh0, ow0, co0, ck;
        bool live;
    };
    auto block_at = [&](int tile, int ck, bool live) {
        Blk r;
        const int t = live ? tile : t_begin;
        const int ct = t % g.co_tiles;
        int q = t / g.co_tiles;
        const int tw = q % g.tiles_w;
        q /= g.tiles_w;
        r.tile = tile;
        r.oh0 = (q % g.tiles_h) * g.TH;
        r.n = q / g.tiles_h;
        r.ow0 = tw * g.TW;
        r.co0 = ct * kBN32;
        r.ck = ck;
        r.live = live;
        return r;
    };
    auto next_of = [&](const Blk &b) {
        if (b.ck + 1 < g.n_chunks) {
            Blk r = b;
            r.ck = b.ck + 1;
            return r;
        }
        return block_at(b.tile + 1, 0, b.live && b.tile + 1 < t_end);
    };

    // ---- window staging ----------------------------------------------------
    // Task t = tid + 512 f: octet o = t&3, row parity (t>>2)&1, column group
    // (t>>3) % ncg, row pair (t>>3) / ncg; fixed per thread, so computed once.
    const int nparts = (((g.FR + 1) / 2) * g.ncg * 8 + kThreads32 - 1) / kThreads32;  // <= kParts
    int tk_o[kParts], tk_cg[kParts], tk_r[kParts];
#pragma unroll
    for (int f = 0; f < kParts; ++f) {
        const int t = tid + f * kThreads32;
        const int rest = t >> 3;
        tk_o[f] = t & 3;
        tk_cg[f] = rest % g.ncg;
        tk_r[f] = 2 * (rest / g.ncg) + ((t >> 2) & 1);
        if (f >= nparts) tk_r[f] = g.FR;  // no rows: idle task
    }
    // A task's 8 loads (channel c of its octet) are issued one at a time so
    // that they can be spread between matrix instructions: fp_off gives the
    // task's first byte offset and the number of its channels to load (0 if
    // none).
    struct LdPlan {
        uint32_t off0;
        int nch;
    };
    auto fp_plan = [&](const Blk &b, int f) {
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo & ~(VEC - 1);  // floor to a multiple of VEC
        const int r = tk_r[f];
        const int ih = b.oh0 * S - s.pad + r;
        const int iw0 = g0 + tk_cg[f] * VEC;
        const bool ok = b.live && r < g.FR && (unsigned)ih < (unsigned)s.H && iw0 >= 0 && iw0 < s.W &&
                        iw0 + VEC - 1 >= iw_lo && iw0 <= iw_lo + g.FC - 1;
        const int ci0 = b.ck * kCK32 + 8 * tk_o[f];
        LdPlan pl;
        pl.off0 = (uint32_t)(((b.n * s.C_in + ci0) * s.H + ih) * s.W + iw0) * 2u;
        pl.nch = ok ? min(8, s.C_in - ci0) : 0;
        return pl;
    };
    auto fp_load_one = [&](const LdPlan &pl, int c) {
        return XV32<VEC>::load(xr, c < pl.nch ? pl.off0 + (uint32_t)(c * s.HW) * 2u : kOOB);
    };
    auto fp_load = [&](const Blk &b, int f, XT (&reg)[8]) {
        const LdPlan pl = fp_plan(b, f);
#pragma unroll
        for (int c = 0; c < 8; ++c) reg[c] = fp_load_one(pl, c);
    };
    // Column j of a task is stored on its own, so that the stores can be
    // spread between matrix instructions; a column outside the window (or
    // of an idle task) goes to this lane's slot of the sink instead of
    // branching.  c0: window column of the task's first element (> -VEC).
    auto fp_c0 = [&](const Blk &b, int f) {
        const int iw_lo = b.ow0 * S - s.pad;
        return (iw_lo & ~(VEC - 1)) + tk_cg[f] * VEC - iw_lo;
    };
    unsigned char *const sink_lane = sink + lane * 16;
    auto fp_store_col = [&](int c0, int f, int j, unsigned char *fp, const XT (&reg)[8]) {
        const int r = tk_r[f];
        const int c = c0 + j;
        // window column c sits at (c mod S) * CS + c / S: the columns of one
        // phase are contiguous, so a tap's columns are consecutive
        const int pos = S == 1 ? c : (c & 1) * g.CS + (c >> 1);
        const bool ok = r < g.FR && c >= 0 && c < g.FC;
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = pair16(reg[2 * d][j >> 1], reg[2 * d + 1][j >> 1], j & 1);
        *(u32x4 *)(ok ? fp + r * g.row_bytes + tk_o[f] * 16 + pos * kRec : sink_lane) = v;
    };
    auto fp_store = [&](const Blk &b, int f, unsigned char *fp, const XT (&reg)[8]) {
        const int c0 = fp_c0(b, f);
#pragma unroll
        for (int j = 0; j < VEC; ++j) fp_store_col(c0, f, j, fp, reg);
    };

    // ---- weight staging: one tap x 128 channels x 4 octets; thread: channel
    // tid >> 2, octet tid & 3 --------------------------------------------------
    const uint32_t w_lane = (uint32_t)((tid >> 2) * g.n_chunks * kT * 64 + (tid & 3) * 16);
    auto w_load = [&](const Blk &b, int tap) {
        const bool ok = b.live && b.co0 + (tid >> 2) < s.C_out;
        return buf_load16(wr, ok ? (uint32_t)((b.co0 * g.n_chunks + b.ck) * kT + tap) * 64u + w_lane : kOOB);
    };
    unsigned char *const w_dst = &wbs[0][0] + (tid >> 2) * kRec + (tid & 3) * 16;

    // ---- per-lane fragment geometry ----------------------------------------
    const int tile_px = g.TH * g.TW;
    uint32_t abase[MB];  // byte address of this lane's pixel record (tap (0,0)), octet hi
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const int px = (wm * MB + b) * 32 + l32;
        const int i = px / g.TW, j = px - (px / g.TW) * g.TW;
        abase[b] = (uint32_t)((px < tile_px ? i * S * g.row_bytes + j * kRec : 0) + hi * 16);
    }
    const uint32_t bbase = (uint32_t)((wn * 32 + l32) * kRec + hi * 16);  // weight record of this lane, octet hi
    const int cs_b = g.CS * kRec;

    f32x16 acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

    // Prologue: the window of the first block and the weights of its first
    // tap group into buffers 0.
    Blk cur = block_at(t_begin, 0, true);
    Blk nxt = next_of(cur);
    XT fpr[kParts][8];
    u32x4 wreg[kGT];
#pragma unroll
    for (int t = 0; t < kGT; ++t) wreg[t] = w_load(cur, t);
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_load(cur, f, fpr[f]);
    });
#pragma unroll
    for (int t = 0; t < kGT; ++t) *(u32x4 *)(w_dst + t * kWTB) = wreg[t];
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_store(cur, f, fps[0], fpr[f]);
    });
    __syncthreads();

    // Group G (three taps; weight buffer G mod 2): request the next group's
    // weights; run the group's 3 x 2 x MB matrix instructions with the
    // fragment reads kDepth ahead of them, and between them write the next
    // group's weights, in a block's first group load the next window, and in
    // its last group write it; barrier.  The order is fixed by scheduling
    // fences: left alone, the compiler sinks each read to just before its
    // use, so that every instruction waits a full LDS round trip, and bunches
    // the loads and stores, which stalls issue.
    constexpr int kM = kGT * 2 * MB;     // matrix instructions per group
    constexpr int kCols = kParts * VEC;  // window columns each thread stores per block
    static_assert(kCols * 5 <= kM && 40 < kM && kParts * 16 <= kM, "staging slots exceed the group");
    bf16x8 fa[kDepth], fb[2];
    // BN factors of this lane's output channel, loaded a tile ahead
    float sc_next, bi_next;
    {
        const int co = cur.co0 + wn * 32 + l32;
        sc_next = co < s.C_out ? scale[co] : 0.f;
        bi_next = co < s.C_out ? bias[co] : 0.f;
    }
    for (int step = 0; step < n_steps; ++step) {
        const unsigned char *fp = fps[step & 1];
        static_for<0, kT / kGT>([&](auto gc) {
            constexpr int gi = decltype(gc)::value;
            constexpr bool last_group = gi == kT / kGT - 1;
            const int wsel = (step * (kT / kGT) + gi) & 1;
            const unsigned char *wb = &wbs[0][0] + wsel * (kGT * kWTB);
            unsigned char *const w_next = w_dst + (wsel ^ 1) * (kGT * kWTB);
#pragma unroll
            for (int t = 0; t < kGT; ++t)
                wreg[t] = gi + 1 < kT / kGT ? w_load(cur, (gi + 1) * kGT + t) : w_load(nxt, t);
            LdPlan lps[kParts];
            if (gi == 0) {
#pragma unroll
                for (int f = 0; f < kParts; ++f) lps[f] = fp_plan(nxt, f);
            }
            int c0s[kParts];
            if (last_group) {
#pragma unroll
                for (int f = 0; f < kParts; ++f) c0s[f] = fp_c0(nxt, f);
            }
            unsigned char *const fp_next = fps[(step + 1) & 1];
            // fragment m of the group: tap gi*3 + m / (2 MB), half (m / MB) % 2,
            // pixel block m % MB; its weight fragment is read with its block 0
            auto issue = [&](auto mc) {
                constexpr int m = decltype(mc)::value;
                if constexpr (m < kM) {
                    constexpr int t = m / (2 * MB), h = (m / MB) % 2, b = m % MB;
                    constexpr int tap = gi * kGT + t, kh = tap / 3, kw = tap % 3;
                    if constexpr (b == 0) fb[(m / MB) % 2] = *(const bf16x8 *)(wb + t * kWTB + bbase + 32 * h);
                    const int toff = kh * g.row_bytes + (kw % S) * cs_b + (kw / S) * kRec;
                    fa[m % kDepth] = *(const bf16x8 *)(fp + abase[b] + toff + 32 * h);
                }
            };
            static_for<0, kDepth>([&](auto mc) { issue(mc); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, kM>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int b = m % MB;
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m % kDepth], fb[(m / MB) % 2], acc[b], 0, 0, 0);
                issue(std::integral_constant<int, m + kDepth>{});
                // next block's window: load q (channel q mod 8 of part q / 8)
                // after matrix instruction 2q + 1 of the first group
                if constexpr (gi == 0 && m % 2 == 1 && m / 2 < kParts * 8) {
                    constexpr int q = m / 2;
                    fpr[q / 8][q % 8] = fp_load_one(lps[q / 8], q % 8);
                }
                // next window: column q after matrix instruction 5q + 1
                if constexpr (last_group && m % 5 == 1 && m / 5 < kCols) {
                    constexpr int q = m / 5;
                    fp_store_col(c0s[q / VEC], q / VEC, q % VEC, fp_next, fpr[q / VEC]);
                }
                // next group's weights: tap t after matrix instruction 20 + 10 t
                if constexpr (m >= 20 && m % 10 == 0 && (m - 20) / 10 < kGT)
                    *(u32x4 *)(w_next + ((m - 20) / 10) * kWTB) = wreg[(m - 20) / 10];
                __builtin_amdgcn_sched_barrier(0);
            });
            __syncthreads();
        });

        if (cur.ck == g.n_chunks - 1) {
            // ---- epilogue for the finished tile ----------------------------
            // Row i = px / TW as (px * ceil(2^20 / TW)) >> 20, exact for the
            // tile's pixels (px < 2 * MB * 32 <= 448, TW <= 448); a division
            // would cost dozens of instructions per store.  (The tile width
            // and its reciprocal pass through an empty asm so that the pixel
            // coordinates are computed here, not hoisted out of the loop into
            // registers the reduction needs.)
            int tw_e = g.TW;
            uint32_t rcp_tw = ((1u << 20) + (uint32_t)g.TW - 1) / (uint32_t)g.TW;
            asm volatile("" : "+s"(tw_e), "+s"(rcp_tw));
            const int co = cur.co0 + wn * 32 + l32;
            const float sc = sc_next, bi = bi_next;
            if (cur.tile + 1 < t_end) {  // the next tile's factors, ahead of its epilogue
                const int co_n = nxt.co0 + wn * 32 + l32;
                sc_next = co_n < s.C_out ? scale[co_n] : 0.f;
                bi_next = co_n < s.C_out ? bias[co_n] : 0.f;
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int px = (wm * MB + b) * 32 + 8 * q + 4 * hi;
                    const int i = (int)(((uint32_t)px * rcp_tw) >> 20), j = px - i * tw_e;
                    const int oh = cur.oh0 + i, ow = cur.ow0 + j;
                    const bool ok = px < tile_px && oh < s.OH && ow < s.OW && co < s.C_out;
                    u32x2 o;
                    const float v0 = acc[b][4 * q], v1 = acc[b][4 * q + 1];
                    const float v2 = acc[b][4 * q + 2], v3 = acc[b][4 * q + 3];
                    if (EPI == kFused) {
                        o.x = pack_bf16x2(bn_silu(v0, sc, bi), bn_silu(v1, sc, bi));
                        o.y = pack_bf16x2(bn_silu(v2, sc, bi), bn_silu(v3, sc, bi));
                    } else {
                        o.x = pack_bf16x2(v0, v1);
                        o.y = pack_bf16x2(v2, v3);
                    }
                    buf_store8(yr, ok ? (uint32_t)(((cur.n * s.C_out + co) * s.OH + oh) * s.OW + ow) * 2u : kOOB,
                               o);
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
            }
        }
        cur = nxt;
        nxt = next_of(cur);
    }
}

struct Config32 {
    int mb, vec;
};
constexpr Config32 kW32v8{7, 8}, kW32v4{7, 4};

// Window geometry of a TH x TW tile; false if it does not fit.
bool make_geo32(const Shape &s, int TH, int TW, const Config32 &cfg, int num_cu, WinGeo *g) {
    g->TH = TH;
    g->TW = TW;
    g->FR = (TH - 1) * s.stride + s.KH;
    g->FC = (TW - 1) * s.stride + s.KW;
    g->CS = (g->FC + s.stride - 1) / s.stride;
    g->FCP = s.stride * g->CS;
    // Row pitch: at least the row's records, and congruent to TW * 80 / S
    // modulo 256 / S bytes, so that output pixel (i, j) of the tile reads a
    // record whose 16-byte bank group is 5 (i TW + j) + (a per-tap constant)
    // mod 16: the 16 consecutive pixels of a half-wave's fragment read hit 16
    // distinct groups of four banks even where they wrap onto the next row.
    const int mod = 256 / s.stride;
    const int want = (TW * kRec / s.stride) % mod;
    int rb = g->FCP * kRec;
    rb += ((want - rb % mod) % mod + mod) % mod;
    g->row_bytes = rb;
    if ((int64_t)g->FR * g->row_bytes > kFpBytes32) return false;
    g->ncg = (g->FC - 1 + cfg.vec - 1) / cfg.vec + 1;
    const int tasks = ((g->FR + 1) / 2) * g->ncg * 8;
    // the next block's window is staged in at most parts_for(vec) parts of 512 tasks
    if (tasks > parts_for(cfg.vec) * kThreads32) return false;
    g->tiles_h = (s.OH + TH - 1) / TH;
    g->tiles_w = (s.OW + TW - 1) / TW;
    g->co_tiles = (s.C_out + kBN32 - 1) / kBN32;
    g->n_tiles = s.N * g->tiles_h * g->tiles_w * g->co_tiles;
    g->n_chunks = (s.C_in + kCK32 - 1) / kCK32;
    g->tiles_per_wg = (g->n_tiles + num_cu - 1) / num_cu;
    g->n_wg = (g->n_tiles + g->tiles_per_wg - 1) / g->tiles_per_wg;
    return true;
}

// The tile with the most output pixels (TW a multiple of 4) whose window
// fits; its pixels fill the 2*MB blocks of 32 as fully as possible.
bool plan32(const Shape &s, const Config32 &cfg, int num_cu, WinGeo *g) {
    const int max_px = 64 * cfg.mb;
    int best = 0;
    WinGeo cand;
    for (int TW = 4; TW <= s.OW && TW <= max_px; TW += 4) {
        int TH = max_px / TW;
        if (TH > s.OH) TH = s.OH;
        for (; TH >= 1; --TH)
            if (make_geo32(s, TH, TW, cfg, num_cu, &cand)) break;
        if (TH < 1) continue;
        // pixels computed per tile, counting the idle part of edge tiles
        const int64_t useful = (int64_t)s.OH * s.OW;
        const int64_t spent = (int64_t)cand.tiles_h * TH * cand.tiles_w * TW;
        const int score = (int)((int64_t)TH * TW * useful / spent);
        if (score > best) {
            best = score;
            *g = cand;
        }
    }
    return best > 0;
}

const Config32 &pick32(const Shape &s) { return s.W % 8 == 0 ? kW32v8 : kW32v4; }

}  // namespace

bool window32_supports(const Shape &s, int dtype) {
    if (dtype != kDtypeBf16 || s.W % 4 != 0 || s.OW % 4 != 0) return false;
    if (s.KH != 3 || s.KW != 3 || (s.stride != 1 && s.stride != 2)) return false;
    if ((uint64_t)s.N * s.C_in * s.HW * 2 > kMaxBufferBytes ||
        (uint64_t)s.N * s.C_out * s.OHW * 2 > kMaxBufferBytes)
        return false;
    if (window_workspace_bytes(s) > kMaxBufferBytes) return false;
    WinGeo g;
    return plan32(s, pick32(s), 256, &g);
}

// Fraction (in 1/1000) of the matrix-core work of a tile spent on real
// output pixels, for the dispatcher.
int window32_efficiency(const Shape &s) {
    WinGeo g;
    if (!plan32(s, pick32(s), 256, &g)) return 0;
    return (int)((int64_t)1000 * g.TH * g.TW / (64 * pick32(s).mb));
}

hipError_t launch_window32(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                           const float *bias, void *y, void *workspace, hipStream_t st, int num_cu) {
    const Config32 &cfg = pick32(s);
    WinGeo g;
    if (!plan32(s, cfg, num_cu, &g)) return hipErrorInvalidValue;
    const hipError_t e = launch_pack_weights(s, w, workspace, st);
    if (e != hipSuccess) return e;
    const dim3 grid(g.n_wg), block(kThreads32);
    auto xx = (const uint16_t *)x;
    auto wp = (const uint16_t *)workspace;
    auto yy = (uint16_t *)y;
#define CBS_W32(C, S_)                                                                                   \
    if (&cfg == &C && s.stride == S_) {                                                                   \
        if (epi == kFused)                                                                                \
            hipLaunchKernelGGL((window32_bf16<C.mb, C.vec, S_, kFused>), grid, block, 0, st, xx, wp, scale, \
                               bias, yy, s, g);                                                          \
        else                                                                                              \
            hipLaunchKernelGGL((window32_bf16<C.mb, C.vec, S_, kConvOnly>), grid, block, 0, st, xx, wp,    \
                               scale, bias, yy, s, g);                                                   \
        return hipGetLastError();                                                                         \
    }
    CBS_W32(kW32v8, 1)
    CBS_W32(kW32v4, 1)
    CBS_W32(kW32v8, 2)
    CBS_W32(kW32v4, 2)
#undef CBS_W32
    return hipErrorInvalidValue;
}

}  // namespace cbs
