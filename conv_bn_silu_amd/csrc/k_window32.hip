// k_window32.hip -- implicit-GEMM convolution on v_mfma_f32_32x32x16_bf16
// for the compute-bound layers (many channels, small images): the input
// window of a tile is staged in LDS once per 32-channel block and reused by
// every kernel tap, as in the 16x16 window kernel, but each wave holds a
// 7 x 2 grid of 32x32 accumulators so that every fragment read from LDS
// feeds several matrix instructions ("Fusing an Epilogue", section "Three
// kernels for one operation": the GEMM kernel has the best arithmetic
// intensity).
//
// Workgroup: 4 waves (one per SIMD) as 2 (pixels) x 2 (channels); tile =
// TH x TW output pixels of one image x 128 output channels; wave (wm, wn)
// owns pixel blocks wm*MB .. wm*MB+MB-1 (32 pixels each, pixel p of the tile
// = row p / TW, column p mod TW) and output channels 64*wn .. +63.
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
// Staging is through registers and runs well ahead of use, so that the
// load latency hides behind the matrix work of one workgroup per CU: a
// tap's weights (128 channels x 64 bytes, 2 x 16 bytes per thread) are
// requested three units ahead (a ring of three register sets; the unit loop
// is unrolled by three), and the next channel block's whole window (up to 3
// parts of 256 tasks, each task 8 channels x VEC columns, transposed with
// byte permutes) is requested at the start of a block and written at its
// end.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"

namespace cbs {

namespace {

constexpr int kThreads32 = 256;
constexpr int kBN32 = 128;            // output channels per tile
constexpr int kCK32 = 32;             // input channels per block
constexpr int kRec = 80;              // bytes per record (64 data + 16 padding)
constexpr int kFpBytes32 = 41 * 1024; // one window buffer
constexpr int kWTB = kBN32 * kRec;    // one weight buffer: one tap x 128 records
constexpr int kParts = 3;             // window parts (256 tasks each) at most

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

// MB: 32-pixel blocks per wave; VEC: input columns per staging load.
template <int MB, int VEC, int EPI>
__global__ __launch_bounds__(kThreads32, 1) void window32_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, WinGeo g) {
    __shared__ __attribute__((aligned(16))) unsigned char fps[2][kFpBytes32];
    __shared__ __attribute__((aligned(16))) unsigned char wbs[2][kWTB];
    typedef typename XV32<VEC>::T XT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, hi = lane >> 5;

    const int t_begin = (int)blockIdx.x * g.tiles_per_wg;
    const int t_end = min(t_begin + g.tiles_per_wg, g.n_tiles);
    if (t_begin >= t_end) return;  // uniform
    const int steps = (t_end - t_begin) * g.n_chunks;  // (tile, channel block) pairs
    const int upt = g.n_chunks * s.T;                  // units (channel block, tap) per tile
    const int upt3 = (upt + 2) / 3 * 3;                // padded to a multiple of 3 (tail units idle)
    const int units = (t_end - t_begin) * upt3;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.HW * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (uint32_t)s.C_out * g.n_chunks * s.T * 64u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);

    struct Tile {
        int n, oh0, ow0, co0;
    };
    auto tile_of = [&](int t) {
        Tile r;
        const int ct = t % g.co_tiles;
        int q = t / g.co_tiles;
        const int tw = q % g.tiles_w;
        q /= g.tiles_w;
        r.oh0 = (q % g.tiles_h) * g.TH;
        r.n = q / g.tiles_h;
        r.ow0 = tw * g.TW;
        r.co0 = ct * kBN32;
        return r;
    };
    // Unit u -> (step, tap); a tile's padding units have none.
    struct Unit {
        int step, tap;
        bool real;
    };
    auto unit_of = [&](int u) {
        const int tl = u / upt3, k = u - tl * upt3;
        Unit r;
        r.real = u < units && k < upt;
        const int kk = k < upt ? k : upt - 1;
        r.step = tl * g.n_chunks + kk / s.T;
        r.tap = kk % s.T;
        return r;
    };

    // ---- window staging ----------------------------------------------------
    // Task t (part f = t / 256): octet o = t&3, row parity (t>>2)&1, column
    // group (t>>3) % ncg, row pair (t>>3) / ncg.
    const int nparts = (((g.FR + 1) / 2) * g.ncg * 8 + kThreads32 - 1) / kThreads32;  // <= kParts
    auto fp_load = [&](int step, int f, XT (&reg)[8]) {
        const int tile = t_begin + step / g.n_chunks;
        const int ck = step % g.n_chunks;
        const bool live = step < steps && f < nparts;
        const Tile tl = tile_of(live ? tile : t_begin);
        const int iw_lo = tl.ow0 * s.stride - s.pad;
        const int g0 = (iw_lo >= 0 ? iw_lo / VEC : -((-iw_lo + VEC - 1) / VEC)) * VEC;
        const int t = tid + f * kThreads32;
        const int rest = t >> 3, o = t & 3;
        const int cg = rest % g.ncg, r = 2 * (rest / g.ncg) + ((t >> 2) & 1);
        const int ih = tl.oh0 * s.stride - s.pad + r;
        const int iw0 = g0 + cg * VEC;
        const bool ok = live && r < g.FR && (unsigned)ih < (unsigned)s.H && iw0 >= 0 && iw0 < s.W &&
                        iw0 + VEC - 1 >= iw_lo && iw0 <= iw_lo + g.FC - 1;
        const uint32_t off0 = (uint32_t)(((tl.n * s.C_in + ck * kCK32 + 8 * o) * s.H + ih) * s.W + iw0) * 2u;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ci = ck * kCK32 + 8 * o + c;
            reg[c] = XV32<VEC>::load(xr, (ok && ci < s.C_in) ? off0 + (uint32_t)(c * s.HW) * 2u : kOOB);
        }
    };
    auto fp_store = [&](int step, int f, unsigned char *fp, const XT (&reg)[8]) {
        if (f >= nparts) return;  // uniform
        const int tile = t_begin + step / g.n_chunks;
        const Tile tl = tile_of(step < steps ? tile : t_begin);
        const int iw_lo = tl.ow0 * s.stride - s.pad;
        const int g0 = (iw_lo >= 0 ? iw_lo / VEC : -((-iw_lo + VEC - 1) / VEC)) * VEC;
        const int t = tid + f * kThreads32;
        const int rest = t >> 3, o = t & 3;
        const int cg = rest % g.ncg, r = 2 * (rest / g.ncg) + ((t >> 2) & 1);
        if (r >= g.FR) return;
        const int c0 = g0 + cg * VEC - iw_lo;  // window column of the group's first element (> -VEC)
        const int c0p = c0 + VEC * s.stride;
        int quo = c0p / s.stride - VEC, rem = c0p - (c0p / s.stride) * s.stride;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int c = c0 + j;
            const int pos = r * g.FCP + rem * g.CS + quo;
            if (++rem == s.stride) {
                rem = 0;
                ++quo;
            }
            if (c < 0 || c >= g.FC) continue;
            u32x4 v;
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = pair16(reg[2 * d][j >> 1], reg[2 * d + 1][j >> 1], j & 1);
            *(u32x4 *)(fp + pos * kRec + o * 16) = v;
        }
    };

    // ---- weight staging: one tap x 128 channels x 4 octets; thread piece q
    // (0, 1): channel (q*256 + tid) >> 2, octet tid & 3 ----------------------
    auto w_load = [&](int u, u32x4 (&reg)[2]) {
        const Unit un = unit_of(u);
        const int tile = t_begin + un.step / g.n_chunks;
        const int ck = un.step % g.n_chunks;
        const int co0 = (tile % g.co_tiles) * kBN32;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int p = q * kThreads32 + tid;
            const int co = co0 + (p >> 2);
            const bool ok = un.real && co < s.C_out;
            reg[q] = buf_load16(wr, ok ? (uint32_t)(((co * g.n_chunks + ck) * s.T + un.tap) * 64 + (p & 3) * 16)
                                       : kOOB);
        }
    };
    auto w_store = [&](unsigned char *wb, const u32x4 (&reg)[2]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int p = q * kThreads32 + tid;
            *(u32x4 *)(wb + (p >> 2) * kRec + (p & 3) * 16) = reg[q];
        }
    };

    // ---- per-lane fragment geometry ----------------------------------------
    const int tile_px = g.TH * g.TW;
    uint32_t abase[MB];  // byte address of this lane's pixel record (tap (0,0)), octet hi
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const int px = (wm * MB + b) * 32 + l32;
        const int i = px / g.TW, j = px - (px / g.TW) * g.TW;
        abase[b] = (uint32_t)((px < tile_px ? i * s.stride * g.FCP + j : 0) * kRec + hi * 16);
    }
    uint32_t bbase[2];  // weight record of this lane, octet hi
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bbase[cb] = (uint32_t)((wn * 64 + 32 * cb + l32) * kRec + hi * 16);

    f32x16 acc[MB][2];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][cb][e] = 0.f;

    // Prologue: window of step 0 and weights of unit 0 into buffers 0;
    // weights of units 1 and 2 in flight in ring slots 1 and 2.
    XT fpr[kParts][8];
    u32x4 wreg[3][2];
    w_load(0, wreg[0]);
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_load(0, f, fpr[f]);
    });
    w_load(1, wreg[1]);
    w_load(2, wreg[2]);
    static_for<0, kParts>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        fp_store(0, f, fps[0], fpr[f]);
    });
    w_store(wbs[0], wreg[0]);
    __syncthreads();

    // Unit u (ring slot u mod 3): request unit u+3's weights; at a block's
    // first tap request the next block's window; the two half-steps (the
    // second's fragments read while the first's 2*MB matrix instructions
    // run); write unit u+1's weights, and after a block's last tap the next
    // window; barrier.
    bf16x8 fa[2][MB], fb[2][2];
    auto run_unit = [&](int u, auto slot_c) {
        constexpr int sl = decltype(slot_c)::value;
        const Unit un = unit_of(u);
        w_load(u + 3, wreg[sl]);
        const bool first = un.real && un.tap == 0;
        const bool last = un.real && un.tap == s.T - 1;
        if (first) {
            static_for<0, kParts>([&](auto fc) {
                constexpr int f = decltype(fc)::value;
                fp_load(un.step + 1, f, fpr[f]);
            });
        }
        if (un.real) {
            const unsigned char *fp = fps[un.step & 1];
            const unsigned char *wb = wbs[u & 1];
            const int kh = un.tap / s.KW, kw = un.tap - kh * s.KW;
            const int toff = (kh * g.FCP + (kw % s.stride) * g.CS + kw / s.stride) * kRec;
            static_for<0, 2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) fb[h][cb] = *(const bf16x8 *)(wb + bbase[cb] + 32 * h);
#pragma unroll
                for (int b = 0; b < MB; ++b) fa[h][b] = *(const bf16x8 *)(fp + abase[b] + toff + 32 * h);
            });
            static_for<0, 2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
#pragma unroll
                for (int b = 0; b < MB; ++b)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[h][b], fb[h][cb], acc[b][cb], 0, 0, 0);
            });
        }
        w_store(wbs[(u + 1) & 1], wreg[(sl + 1) % 3]);
        if (last) {
            static_for<0, kParts>([&](auto fc) {
                constexpr int f = decltype(fc)::value;
                fp_store(un.step + 1, f, fps[(un.step + 1) & 1], fpr[f]);
            });
        }
        __syncthreads();
    };

    for (int tile = t_begin; tile < t_end; ++tile) {
        const int u0 = (tile - t_begin) * upt3;
        for (int k = 0; k < upt3; k += 3) {
            run_unit(u0 + k, std::integral_constant<int, 0>{});
            run_unit(u0 + k + 1, std::integral_constant<int, 1>{});
            run_unit(u0 + k + 2, std::integral_constant<int, 2>{});
        }

        // ---- epilogue for the finished tile --------------------------------
        // (The tile width is passed through an empty asm so that the pixel
        // coordinates below are computed here, not hoisted out of the loop
        // into registers the reduction needs.)
        int tw_e = g.TW;
        asm volatile("" : "+s"(tw_e));
        const Tile tl = tile_of(tile);
        float sc[2], bi[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int co = tl.co0 + wn * 64 + 32 * cb + l32;
            sc[cb] = co < s.C_out ? scale[co] : 0.f;
            bi[cb] = co < s.C_out ? bias[co] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int px = (wm * MB + b) * 32 + 8 * q + 4 * hi;
                const int i = px / tw_e, j = px - i * tw_e;
                const int oh = tl.oh0 + i, ow = tl.ow0 + j;
                const bool pok = px < tile_px && oh < s.OH && ow < s.OW;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int co = tl.co0 + wn * 64 + 32 * cb + l32;
                    const bool ok = pok && co < s.C_out;
                    u32x2 o;
                    const float v0 = acc[b][cb][4 * q], v1 = acc[b][cb][4 * q + 1];
                    const float v2 = acc[b][cb][4 * q + 2], v3 = acc[b][cb][4 * q + 3];
                    if (EPI == kFused) {
                        o.x = pack_bf16x2(bn_silu(v0, sc[cb], bi[cb]), bn_silu(v1, sc[cb], bi[cb]));
                        o.y = pack_bf16x2(bn_silu(v2, sc[cb], bi[cb]), bn_silu(v3, sc[cb], bi[cb]));
                    } else {
                        o.x = pack_bf16x2(v0, v1);
                        o.y = pack_bf16x2(v2, v3);
                    }
                    buf_store8(yr, ok ? (uint32_t)(((tl.n * s.C_out + co) * s.OH + oh) * s.OW + ow) * 2u : kOOB, o);
                }
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[b][cb][e] = 0.f;
        }
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
    // the next block's window is staged in at most kParts parts of 256 tasks
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
#define CBS_W32(C)                                                                                       \
    if (&cfg == &C) {                                                                                     \
        if (epi == kFused)                                                                                \
            hipLaunchKernelGGL((window32_bf16<C.mb, C.vec, kFused>), grid, block, 0, st, xx, wp, scale,     \
                               bias, yy, s, g);                                                          \
        else                                                                                              \
            hipLaunchKernelGGL((window32_bf16<C.mb, C.vec, kConvOnly>), grid, block, 0, st, xx, wp,        \
                               scale, bias, yy, s, g);                                                   \
        return hipGetLastError();                                                                         \
    }
    CBS_W32(kW32v8)
    CBS_W32(kW32v4)
#undef CBS_W32
    return hipErrorInvalidValue;
}

}  // namespace cbs
