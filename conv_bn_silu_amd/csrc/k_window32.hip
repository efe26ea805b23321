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
// Reduction order: channel block (32 channels), then the tap (a "unit"),
// then two 16-channel halves.  LDS holds two window buffers (this channel
// block and the next) and two weight buffers (this tap and the next); one
// barrier per unit.  A record holds 32 channels of one input position
// (window) or one output channel (weights) in 64 bytes, padded to 80: with 5
// 16-byte slots per record, 16 lanes reading one slot of 16 consecutive
// records hit 16 distinct bank groups of gfx950's 64-bank LDS, and a
// fragment -- 8 consecutive channels of one pixel or one output channel per
// lane -- is one ds_read_b128 whose per-tap part of the address is a
// uniform offset.
//
// Staging is through registers and runs well ahead of use: a tap's weights
// (128 channels x 64 bytes, 16 bytes per thread) are requested three units
// ahead (a ring of three register sets), and the next channel block's whole
// window (up to 2 parts of 512 tasks, each task 8 channels x VEC columns,
// transposed with byte permutes) is requested at the start of a block and
// written at its end.  The nine taps are unrolled with the stride fixed at
// compile time, and blocks advance by counters, so that a unit costs no
// integer division: the scalar unit, shared by both waves of a SIMD, would
// otherwise issue more instructions per unit than the matrix core runs.
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
constexpr int kWTB = kBN32 * kRec;    // one weight buffer: one tap x 128 records
constexpr int kParts = 2;             // window parts (512 tasks each) at most

// Calls f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ uint32_t pair16(uint32_t lo_word, uint32_t hi_word, int h) {
    return h == 0 ? ((lo_word & 0xFFFFu) | (hi_word << 16)) : ((lo_word >> 16) | (hi_word & 0xFFFF0000u));
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
    __shared__ __attribute__((aligned(16))) unsigned char wbs[2][kWTB];
    typedef typename XV32<VEC>::T XT;
    constexpr int kT = 9;  // taps

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, hi = lane >> 5;

    const int t_begin = (int)blockIdx.x * g.tiles_per_wg;
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
    auto fp_load = [&](const Blk &b, int f, XT (&reg)[8]) {
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo & ~(VEC - 1);  // floor to a multiple of VEC
        const int r = tk_r[f];
        const int ih = b.oh0 * S - s.pad + r;
        const int iw0 = g0 + tk_cg[f] * VEC;
        const bool ok = b.live && r < g.FR && (unsigned)ih < (unsigned)s.H && iw0 >= 0 && iw0 < s.W &&
                        iw0 + VEC - 1 >= iw_lo && iw0 <= iw_lo + g.FC - 1;
        const int ci0 = b.ck * kCK32 + 8 * tk_o[f];
        const uint32_t off0 = (uint32_t)(((b.n * s.C_in + ci0) * s.H + ih) * s.W + iw0) * 2u;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            reg[c] = XV32<VEC>::load(xr, (ok && ci0 + c < s.C_in) ? off0 + (uint32_t)(c * s.HW) * 2u : kOOB);
    };
    auto fp_store = [&](const Blk &b, int f, unsigned char *fp, const XT (&reg)[8]) {
        const int r = tk_r[f];
        if (r >= g.FR) return;
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo & ~(VEC - 1);
        const int c0 = g0 + tk_cg[f] * VEC - iw_lo;  // window column of the group's first element (> -VEC)
        unsigned char *row = fp + (r * g.FCP) * kRec + tk_o[f] * 16;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int c = c0 + j;
            if (c < 0 || c >= g.FC) continue;
            // window column c sits at (c mod S) * CS + c / S: the columns of
            // one phase are contiguous, so a tap's columns are consecutive
            const int pos = S == 1 ? c : (c & 1) * g.CS + (c >> 1);
            u32x4 v;
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = pair16(reg[2 * d][j >> 1], reg[2 * d + 1][j >> 1], j & 1);
            *(u32x4 *)(row + pos * kRec) = v;
        }
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
        abase[b] = (uint32_t)((px < tile_px ? i * S * g.FCP + j : 0) * kRec + hi * 16);
    }
    const uint32_t bbase = (uint32_t)((wn * 32 + l32) * kRec + hi * 16);  // weight record of this lane, octet hi
    const int fcp_b = g.FCP * kRec, cs_b = g.CS * kRec;

    f32x16 acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

    // Prologue: the window of the first block and the weights of its tap 0
    // into buffers 0; taps 1 and 2 in flight in ring slots 1 and 2.
    Blk cur = block_at(t_begin, 0, true);
    Blk nxt = next_of(cur);
    XT fpr[kParts][8];
    u32x4 wreg[3];
    wreg[0] = w_load(cur, 0);
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_load(cur, f, fpr[f]);
    });
    wreg[1] = w_load(cur, 1);
    wreg[2] = w_load(cur, 2);
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_store(cur, f, fps[0], fpr[f]);
    });
    *(u32x4 *)w_dst = wreg[0];
    __syncthreads();

    // Unit (block, tap), ring slot tap mod 3, weight buffer (unit index) mod 2
    // = (step + tap) mod 2 as nine is odd: request the weights three units
    // ahead; at tap 0 request the next block's window; the two half-steps
    // (the second's fragments read while the first's MB matrix instructions
    // run); write the next unit's weights, and after tap 8 the next window;
    // barrier.
    bf16x8 fa[2][MB], fb[2];
    for (int step = 0; step < n_steps; ++step) {
        const unsigned char *fp = fps[step & 1];
        static_for<0, kT>([&](auto tc) {
            constexpr int tap = decltype(tc)::value;
            constexpr int sl = tap % 3;
            wreg[sl] = tap + 3 < kT ? w_load(cur, tap + 3) : w_load(nxt, tap + 3 - kT);
            if (tap == 0) {
                static_for<0, kParts>([&](auto fc) {
                    constexpr int f = decltype(fc)::value;
                    fp_load(nxt, f, fpr[f]);
                });
            }
            const int wsel = (step + tap) & 1;
            const unsigned char *wb = &wbs[0][0] + wsel * kWTB;
            constexpr int kh = tap / 3, kw = tap % 3;
            const int toff = kh * fcp_b + (kw % S) * cs_b + (kw / S) * kRec;
            static_for<0, 2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
                fb[h] = *(const bf16x8 *)(wb + bbase + 32 * h);
#pragma unroll
                for (int b = 0; b < MB; ++b) fa[h][b] = *(const bf16x8 *)(fp + abase[b] + toff + 32 * h);
            });
            static_for<0, 2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[h][b], fb[h], acc[b], 0, 0, 0);
            });
            *(u32x4 *)(w_dst + (wsel ^ 1) * kWTB) = wreg[(sl + 1) % 3];
            if (tap == kT - 1) {
                static_for<0, kParts>([&](auto fc) {
                    constexpr int f = decltype(fc)::value;
                    fp_store(nxt, f, fps[(step + 1) & 1], fpr[f]);
                });
            }
            __syncthreads();
        });

        if (cur.ck == g.n_chunks - 1) {
            // ---- epilogue for the finished tile ----------------------------
            // (The tile width is passed through an empty asm so that the pixel
            // coordinates below are computed here, not hoisted out of the loop
            // into registers the reduction needs.)
            int tw_e = g.TW;
            asm volatile("" : "+s"(tw_e));
            const int co = cur.co0 + wn * 32 + l32;
            const float sc = co < s.C_out ? scale[co] : 0.f;
            const float bi = co < s.C_out ? bias[co] : 0.f;
#pragma unroll
            for (int b = 0; b < MB; ++b) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int px = (wm * MB + b) * 32 + 8 * q + 4 * hi;
                    const int i = px / tw_e, j = px - i * tw_e;
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
    if (g->FCP % 2 == 0) g->FCP += 1;
    if ((int64_t)g->FR * g->FCP * kRec > kFpBytes32) return false;
    g->ncg = (g->FC - 1 + cfg.vec - 1) / cfg.vec + 1;
    const int tasks = ((g->FR + 1) / 2) * g->ncg * 8;
    // the next block's window is staged in at most kParts parts of 512 tasks
    if (tasks > kParts * kThreads32) return false;
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
