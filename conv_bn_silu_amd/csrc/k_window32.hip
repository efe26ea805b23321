// k_window32.hip -- implicit-GEMM 3x3 convolution on v_mfma_f32_32x32x16_bf16
// for the compute-bound layers (many channels, small images): the GEMM kernel
// of "Fusing an Epilogue" (section "Three kernels for one operation": the
// kernel that reuses each loaded value the most), with the input window of a tile
// staged in LDS once per 16-channel chunk and reused by all nine taps, and
// the weights read straight from their OIHW layout (no reordered copy).
//
// GEMM view: rows are the output pixels of a tile (TH x TW of one image, in
// 32-pixel blocks; pixel p of the tile is row p / TW, column p mod TW),
// columns are 128 output channels (four 32-channel blocks), and the
// reduction runs over (16-channel chunk, tap, channel).  For a chunk the k
// values of tap (kh, kw) at output pixel (i, j) are the 16 channels of input
// position (i*S + kh, j*S + kw): staged once, the window serves every tap.
//
// Work split.  One workgroup of 4 waves per CU (one wave per SIMD), with 13
// pixel blocks (up to 416 pixels: a 400-pixel image fills 12.5 of them) x 4
// channel blocks = 52 cells of 32x32 per tile.  Wave (h, c) takes channel
// blocks 2c and 2c+1 and half h of the pixel blocks in a diagonal split:
// numbering the 26 cells of those two channel blocks pixel-block-major, half
// 0 is the first 13 and half 1 the rest.  Each half is 7 pixel blocks x 2
// channel blocks minus one corner, so every wave runs 13 matrix instructions
// per k step and reads 7 + 2 fragments for them (each pixel fragment feeds
// two instructions, each weight fragment six or seven).  Half 1 walks its
// pixel blocks from the last one down and swaps its two channel blocks, so
// that its missing corner is the same local cell as half 0's and the skip is
// fixed at compile time.  All 13 accumulators of a wave stay in registers
// for the whole reduction.
//
// LDS, double buffered by chunk:
//  * weights: [tap][channel octet][output channel] records of 16 bytes (8
//    input channels of one output channel and tap): the fragment reads and
//    the staging writes both put 16 lanes on 16 consecutive output channels,
//    16 distinct bank groups.
//  * window: [channel octet][row][position] records of 16 bytes (8 channels
//    of one input position).  For stride 2 the columns of a row are stored
//    even ones first, then odd ones, so that a tap's columns are consecutive.
//    The row pitch R (records) satisfies S*R = TW (mod 16): the 16 pixels of
//    a half-wave's fragment read then hit 16 distinct bank groups even where
//    they wrap onto the next output row.
// One barrier per chunk.  During chunk c the next chunk's weights and window
// are loaded into registers (issued early in the chunk, spread between the
// matrix instructions), transposed with byte permutes and written to the
// other buffer late in the chunk; the barrier sits inside the chunk's last k
// step, after which the next chunk's first fragments are read.  The
// fragments of k step t+1 are read during k step t.
//
// Window staging: a task is 8 channels x 8 columns of one input row -- eight
// 16-byte loads, one per channel -- transposed into 8 position records with
// byte permutes.  Where W = 4 mod 8 the rows start on 8-byte boundaries and a
// row's last group reads 4 elements of the next row; those columns are zeroed
// when the records are formed (zeroing them at the load would make every
// load wait for its data on the spot).
//
// Weight staging: each wave loads the OIHW rows of its 32 output channels
// for the chunk (16 channels x 9 taps = 288 contiguous bytes each) with
// coalesced 16-byte loads -- neighbouring lanes read neighbouring pieces --
// into a raw LDS area of its own; lane (channel o, octet q) then reads back
// the 72 weights w[co][ci0+8q .. +7][0..8] and rearranges them into nine tap
// records (36 byte permutes).
//
// Epilogue: folded BN + SiLU on the accumulators, bf16, 8-byte stores of
// four consecutive pixels of one channel; the BN factors of the next tile are
// loaded a tile ahead.
#include <type_traits>

#include "cbs_device.h"
#include "cbs_launch.h"


namespace cbs {

namespace {

constexpr int kThreads32 = 256;
constexpr int kBN32 = 128;                   // output channels per tile
constexpr int kCK32 = 16;                    // input channels per chunk
constexpr int kPW = 128;                     // weight records per (tap, octet)
constexpr int kWBytes = 9 * 2 * kPW * 16;    // one chunk's weights, tap-major: 36,864 bytes
constexpr int kRawPitch = 19 * 16;           // bytes per output channel in the raw weight area
constexpr int kRawWave = 32 * kRawPitch;     // one wave's raw weights: 9,728 bytes
constexpr int kWinBytes = (160 * 1024 - 2 * kWBytes - 4 * kRawWave) / 2;  // one chunk's window, at most
constexpr int kMaxTasks32 = 2;               // window staging tasks per thread, at most
constexpr int kVec = 8;                      // input columns per window staging load

// Bytes per channel-octet plane of the window: FR rows, padded by one record
// when the plane's record count is a multiple of 4.  A staging write of 16
// lanes covers 2 octets x 8 (row, column group) pairs at one column, whose
// records all fall on 4 residues mod 16 within a plane (the row pitch is
// fixed by the fragment reads); an octet offset off those residues puts the
// two octets on distinct banks, halving the conflict.  Fragment reads stay
// within one plane.
__host__ __device__ constexpr int win_plane_bytes(int FR, int row_bytes) {
    return ((FR * row_bytes) >> 4) % 4 == 0 ? FR * row_bytes + 16 : FR * row_bytes;
}

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

// Element e (0..71) of a thread's 72 weights w[co][ci0 + e/9][e%9], held as
// nine 16-byte loads: its 32-bit word and half.
__device__ __forceinline__ uint32_t w_word(const u32x4 (&wr)[9], int e) { return wr[e >> 3][(e >> 1) & 3]; }

// S: stride (1 or 2); TASKS: window staging tasks per thread (1 or 2).
template <int S, int TASKS, int EPI>
__global__ __launch_bounds__(kThreads32, 1) void window32_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ scale,
    const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, WinGeo g) {
    // window buffers first, so that a window fragment's address is a
    // register plus an immediate offset below 64 KiB
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kWinBytes + 2 * kWBytes + 4 * kRawWave];
    unsigned char *const win = lds;
    unsigned char *const wts = lds + 2 * kWinBytes;
    constexpr int VEC = kVec;
    constexpr int kTasks32 = TASKS;
    typedef u32x4 XT;
    constexpr int PBX = 13;             // pixel blocks per tile
    constexpr int NC = 13;              // cells (matrix instructions per k step) per wave
    constexpr int kT = 9;               // taps

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in scalar registers
    const int hf = wave & 1, cp = wave >> 1;
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

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)s.N * s.C_in * s.HW * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)s.C_out * s.K * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)s.N * s.C_out * s.OHW * 2u);
    const int R = g.row_bytes >> 4;                // window row pitch in records
    const int plane_bytes = win_plane_bytes(g.FR, g.row_bytes);  // one channel octet of the window

    // A step: one 16-channel chunk of one tile.
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

    // ---- weight staging: wave w stages output channels co0 + 32w .. +31 ------
    // Loads: lane l of load q takes 16-byte piece 64q + l of the wave's 32
    // OIHW rows of this chunk (18 pieces per output channel: 16 channels x 9
    // taps), so each load reads a few contiguous row segments.  The pieces go
    // to the wave's own raw area (rows padded to 19 records), and lane
    // (channel l & 31, octet l >> 5) reads back its 144-byte run, permutes it
    // into tap records and writes them tap-major.  All within one wave, whose
    // LDS operations run in order, so no barrier is needed for the raw area.
    unsigned char *const raw_w = lds + 2 * kWinBytes + 2 * kWBytes + wave * kRawWave;
    auto w_load = [&](const Blk &b, int q) {
        // With two staging tasks per thread every register is taken: there
        // the lane index is produced afresh (volatile asm, not hoisted) so
        // that no per-lane offset is held across the loops.
        int ln = lane;
        if constexpr (TASKS == 2) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const int P = 64 * q + ln, row = P / 18, pc = P - row * 18;
        const int co = b.co0 + 32 * wave + row;
        const bool ok = b.live & (co < s.C_out) & (b.ck * kCK32 + (pc >= 9 ? 8 : 0) < s.C_in);
        // the offset is formed for every lane and then selected: left to
        // itself the compiler guards the multiply with a branch per load
        uint32_t off = (uint32_t)((co * s.C_in + b.ck * kCK32) * 18 + pc * 16);
        asm("" : "+v"(off));
        return buf_load16(wr, ok ? off : kOOB);
    };
    auto w_raw_store = [&](int q, const u32x4 &v) {
        const int P = 64 * q + lane, row = P / 18, pc = P - row * 18;
        *(u32x4 *)(raw_w + row * kRawPitch + pc * 16) = v;
    };
    const int tco = lane & 31, toct = lane >> 5;
    auto w_raw_load = [&](int q) { return *(const u32x4 *)(raw_w + tco * kRawPitch + toct * 144 + 16 * q); };
    unsigned char *const w_dst = wts + (toct * kPW + 32 * wave + tco) * 16;
    // record of tap t: 8 input channels c = 0..7, element c*9 + t of the run
    auto w_record = [&](const u32x4 (&wrg)[9], int t) {
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int e0 = (2 * d) * 9 + t, e1 = e0 + 9;
            v[d] = __builtin_amdgcn_perm(w_word(wrg, e1), w_word(wrg, e0),
                                         ((e0 & 1) ? 0x0302u : 0x0100u) | ((e1 & 1) ? 0x07060000u : 0x05040000u));
        }
        return v;
    };

    // ---- window staging: task t = tid + 256 f: octet t&1, column group
    // (t>>1) % ncg, row (t>>1) / ncg; fixed per thread ----------------------
    int tk_o[kTasks32], tk_cg[kTasks32], tk_r[kTasks32];
#pragma unroll
    for (int f = 0; f < kTasks32; ++f) {
        const int t = tid + f * kThreads32;
        tk_o[f] = t & 1;
        tk_cg[f] = (t >> 1) % g.ncg;
        tk_r[f] = (t >> 1) / g.ncg;
        if (tk_r[f] > g.FR) tk_r[f] = g.FR;  // no row: idle task
    }
    struct LdPlan {
        uint32_t off0;
        int nch;    // channels of the octet to load (0 if none)
    };
    auto fp_plan = [&](const Blk &b, int f) {
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo >= 0 ? iw_lo & ~(VEC - 1) : -((-iw_lo + VEC - 1) & ~(VEC - 1));
        const int r = tk_r[f];
        const int ih = b.oh0 * S - s.pad + r;
        const int iw0 = g0 + tk_cg[f] * VEC;
        const bool ok = b.live & (r < g.FR) & ((unsigned)ih < (unsigned)s.H) & (iw0 >= 0) & (iw0 < s.W) &
                        (iw0 <= iw_lo + g.FC - 1);
        const int ci0 = b.ck * kCK32 + 8 * tk_o[f];
        LdPlan pl;
        pl.off0 = (uint32_t)(((b.n * s.C_in + ci0) * s.H + ih) * s.W + iw0) * 2u;
        pl.nch = ok ? min(8, s.C_in - ci0) : 0;
        return pl;
    };
    // 16-byte loads of 8 columns; rows of W = 4 mod 8 start 8-byte aligned,
    // and the last group of such a row reads 4 elements of the next row,
    // which are zeroed here
    auto fp_load_one = [&](const LdPlan &pl, int c) {
        return buf_load16(xr, c < pl.nch ? pl.off0 + (uint32_t)(c * s.HW) * 2u : kOOB);
    };
    auto fp_c0 = [&](const Blk &b, int f) {  // window column of the task's first element (> -VEC)
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo >= 0 ? iw_lo & ~(VEC - 1) : -((-iw_lo + VEC - 1) & ~(VEC - 1));
        return g0 + tk_cg[f] * VEC - iw_lo;
    };
    // masked-off stores go to the wave's raw weight area, idle while the
    // window is written
    unsigned char *const sink_lane = raw_w + lane * 16;
    // Column j of task f: record of its 8 channels at that column, to window
    // position (row r, column c) of buffer `buf`, or to the sink.
    auto fp_edge = [&](const Blk &b, int f) {  // the task's group runs past the row end
        const int iw_lo = b.ow0 * S - s.pad;
        const int g0 = iw_lo >= 0 ? iw_lo & ~(VEC - 1) : -((-iw_lo + VEC - 1) & ~(VEC - 1));
        return g0 + tk_cg[f] * VEC + VEC > s.W;
    };
    auto fp_store_col = [&](int c0, bool edge_f, int f, int j, unsigned char *buf, const XT (&reg)[8]) {
        const int r = tk_r[f];
        const int c = c0 + j;
        const int pos = S == 1 ? c : (c & 1) * g.CS + (c >> 1);
        const bool ok = r < g.FR && c >= 0 && c < g.FC;
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = pair16(reg[2 * d][j >> 1], reg[2 * d + 1][j >> 1], j & 1);
        if (j >= 4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = edge_f ? 0u : v[d];
        }
        *(u32x4 *)(ok ? buf + tk_o[f] * plane_bytes + (r * R + pos) * 16 : sink_lane) = v;
    };

    // ---- per-lane fragment geometry ----------------------------------------
    const int tile_px = g.TH * g.TW;
    uint32_t abase[7];  // window byte offset of this lane's pixel at tap (0, 0), octet hi
#pragma unroll
    for (int lb = 0; lb < 7; ++lb) {
        const int pb = hf == 0 ? lb : PBX - 1 - lb;
        const int px = pb * 32 + l32;
        const int i = px / g.TW, j = px - (px / g.TW) * g.TW;
        abase[lb] = (uint32_t)(hi * plane_bytes + (px < tile_px ? (S * i * R + j) * 16 : 0));
    }
    int cbk[2];  // channel block of local column cs
    cbk[0] = 2 * cp + (hf == 0 ? 0 : 1);
    cbk[1] = 2 * cp + (hf == 0 ? 1 : 0);
    uint32_t bbase[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) bbase[cs] = (uint32_t)((hi * kPW + cbk[cs] * 32 + l32) * 16);
    int toff[kT];  // window byte offset of tap (kh, kw)
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        const int kh = t / 3, kw = t % 3;
        toff[t] = (kh * R + (S == 1 ? kw : (kw & 1) * g.CS + (kw >> 1))) * 16;
    }

    // ---- prologue: the first step's weights and window into buffers 0 ------
    Blk cur = block_at(t_begin, 0, true);
    Blk nxt = next_of(cur);
    u32x4 wrg[9];
    XT fpr[kTasks32][8];
    {
#pragma unroll
        for (int q = 0; q < 9; ++q) wrg[q] = w_load(cur, q);
#pragma unroll
        for (int f = 0; f < kTasks32; ++f) {
            const LdPlan pl = fp_plan(cur, f);
#pragma unroll
            for (int c = 0; c < 8; ++c) fpr[f][c] = fp_load_one(pl, c);
        }
#pragma unroll
        for (int q = 0; q < 9; ++q) w_raw_store(q, wrg[q]);
#pragma unroll
        for (int q = 0; q < 9; ++q) wrg[q] = w_raw_load(q);
#pragma unroll
        for (int t = 0; t < kT; ++t) *(u32x4 *)(w_dst + t * (2 * kPW * 16)) = w_record(wrg, t);
#pragma unroll
        for (int f = 0; f < kTasks32; ++f) {
            const int c0 = fp_c0(cur, f);
            const bool e = fp_edge(cur, f);
#pragma unroll
            for (int j = 0; j < VEC; ++j) fp_store_col(c0, e, f, j, win, fpr[f]);
        }
    }
    __syncthreads();

    // Fragments: a pixel fragment is read for the next k step right after
    // this step's last instruction that uses it (single buffer); the weight
    // fragments, used all through a step, alternate between two sets by the
    // parity of the k step.
    bf16x8 fa[7], fb[2][2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) fb[0][cs] = *(const bf16x8 *)(wts + bbase[cs]);
#pragma unroll
    for (int lb = 0; lb < 7; ++lb) fa[lb] = *(const bf16x8 *)(win + abase[lb] + toff[0]);

    // BN factors of this lane's two output channels, loaded a tile ahead
    // (buffer loads: zero past C_out, without a branch)
    const __amdgpu_buffer_rsrc_t scr = make_rsrc(scale, (uint32_t)s.C_out * 4u);
    const __amdgpu_buffer_rsrc_t bir = make_rsrc(bias, (uint32_t)s.C_out * 4u);
    float sc_next[2], bi_next[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
        const uint32_t off = (uint32_t)(cur.co0 + cbk[cs] * 32 + l32) * 4u;
        sc_next[cs] = __builtin_bit_cast(float, buf_load4(scr, off));
        bi_next[cs] = __builtin_bit_cast(float, buf_load4(bir, off));
    }

    // Slots of one chunk: slot z = k * NC + m follows matrix instruction m of
    // k step k.  The next step's staging sits at fixed slots: weight loads in
    // k step 0, window loads in steps 1-2, the raw weights written in step 4
    // (four steps after their loads) and read back right after, tap records
    // written in step 5, window records in steps 6-7, the barrier after
    // instruction 1 of step 8.
    constexpr int zWLoad = 0;
    constexpr int zXLoad = NC + 2;
    constexpr int zWRaw = 4 * NC;
    constexpr int zWBack = 4 * NC + 9;
    constexpr int zWStore = 5 * NC + 5;
    constexpr int zXStore = 6 * NC + 2;
    constexpr int zBarrier = 8 * NC + 1;
    static_assert(zWLoad + 9 <= zWRaw && zWRaw + 9 <= zWBack && zWBack + 9 <= zWStore &&
                      zXLoad + 8 * kTasks32 <= zWRaw && zWStore + 9 <= zXStore &&
                      zXStore + kTasks32 * VEC <= zBarrier, "staging slots overlap");
    constexpr int kLastA6 = 12;  // instruction of the last use of pixel fragment 6

    f32x16 acc[NC];

    // One chunk; PAR = step parity = LDS buffer of this chunk.
    auto chunk = [&](auto par_c) {
        constexpr int PAR = decltype(par_c)::value;
        // Fragment-read bases, made opaque here so that the address sums of
        // the reads are formed next to the reads, not hoisted out of the loop
        // into registers of their own.
        uint32_t ab[7], bcur[2], bnxt[2];
#pragma unroll
        for (int lb = 0; lb < 7; ++lb) {
            ab[lb] = abase[lb];
            asm volatile("" : "+v"(ab[lb]));
        }
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            bcur[cs] = 2 * kWinBytes + PAR * kWBytes + bbase[cs];
            bnxt[cs] = 2 * kWinBytes + (PAR ^ 1) * kWBytes + bbase[cs];
            asm volatile("" : "+v"(bcur[cs]), "+v"(bnxt[cs]));
        }
        unsigned char *const w_next = w_dst + (PAR ^ 1) * kWBytes;
        unsigned char *const x_next = win + (PAR ^ 1) * kWinBytes;
        LdPlan lps[kTasks32];
        int c0s[kTasks32];
        bool eds[kTasks32];
        static_for<0, kT>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr int fs = (PAR + k) & 1, fn = fs ^ 1;  // weight fragment sets: this step, next step
            constexpr bool last = k + 1 == kT;              // the next step is the next chunk's tap 0
            constexpr int ntap = last ? 0 : k + 1;
            constexpr int xoff = (last ? PAR ^ 1 : PAR) * kWinBytes;
            auto rdB = [&](int cs) {
                fb[fn][cs] = *(const bf16x8 *)(lds + (last ? bnxt[cs] : bcur[cs]) + ntap * (2 * kPW * 16));
            };
            auto rdA = [&](int lb) { fa[lb] = *(const bf16x8 *)(lds + xoff + (ab[lb] + (uint32_t)toff[ntap])); };
            if constexpr (k == 1) {
#pragma unroll
                for (int f = 0; f < kTasks32; ++f) lps[f] = fp_plan(nxt, f);
            }
            if constexpr (k == 6) {
#pragma unroll
                for (int f = 0; f < kTasks32; ++f) {
                    c0s[f] = fp_c0(nxt, f);
                    eds[f] = fp_edge(nxt, f);
                }
            }
            static_for<0, NC>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int lb = m >> 1, cs = m & 1;
                constexpr int z = k * NC + m;
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[lb], fb[fs][cs], acc[m], 0, 0, 0);
                if constexpr (z == zBarrier) __syncthreads();
                if constexpr (m == 1) {
                    rdB(0);
                    rdB(1);
                }
                if constexpr (m % 2 == 1 && lb < 6) rdA(lb);
                if constexpr (m == kLastA6) rdA(6);
                if constexpr (z >= zWLoad && z < zWLoad + 9) wrg[z - zWLoad] = w_load(nxt, z - zWLoad);
                if constexpr (z >= zWRaw && z < zWRaw + 9) w_raw_store(z - zWRaw, wrg[z - zWRaw]);
                if constexpr (z >= zWBack && z < zWBack + 9) wrg[z - zWBack] = w_raw_load(z - zWBack);
                if constexpr (z >= zXLoad && z < zXLoad + 8 * kTasks32) {
                    constexpr int q = z - zXLoad;
                    fpr[q / 8][q % 8] = fp_load_one(lps[q / 8], q % 8);
                }
                if constexpr (z >= zWStore && z < zWStore + 9) {
                    constexpr int t = z - zWStore;
                    *(u32x4 *)(w_next + t * (2 * kPW * 16)) = w_record(wrg, t);
                }
                if constexpr (z >= zXStore && z < zXStore + kTasks32 * VEC) {
                    constexpr int q = z - zXStore;
                    fp_store_col(c0s[q / VEC], eds[q / VEC], q / VEC, q % VEC, x_next, fpr[q / VEC]);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });

        cur = nxt;
        nxt = next_of(cur);
    };

    // Tiles; per tile the accumulators start at zero, the chunks run in
    // pairs (their count is even: a chunk past C_in adds zeros), and the
    // epilogue follows.  (Zeroing the accumulators at the top of the tile
    // loop, not at the end of an epilogue inside the chunk loop, keeps them
    // in the accumulation registers across the loop.)
    for (int tile = t_begin; tile < t_end; ++tile) {
        const Blk tb = block_at(tile, 0, true);
#pragma unroll
        for (int m = 0; m < NC; ++m)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;
        for (int pr = 0; pr < g.n_chunks; pr += 2) {
            chunk(std::integral_constant<int, 0>{});
            chunk(std::integral_constant<int, 1>{});
        }

        // ---- epilogue ----------------------------------------------------------
        // Row i = px / TW as (px * ceil(2^20 / TW)) >> 20, exact for the
        // tile's pixels (px < 416, TW <= 416).  The tile width, its
        // reciprocal and the lane's own coordinates pass through an empty asm
        // so that every pixel and channel index of the stores is computed
        // here, not hoisted out of the loops into registers the reduction
        // needs.  The lane index is recomputed here (mbcnt, in a volatile asm
        // that cannot be hoisted) rather than kept from the prologue: a value
        // live across the whole tile loop is one register more than the
        // two-task staging leaves free.
        int tw_e = g.TW;
        uint32_t rcp_tw = ((1u << 20) + (uint32_t)g.TW - 1) / (uint32_t)g.TW;
        int lane_e, hf_e = hf;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
        asm volatile("" : "+s"(tw_e), "+s"(rcp_tw), "+v"(lane_e), "+s"(hf_e));
        const int l32_e = lane_e & 31, hi_e = lane_e >> 5;
        float sc[2], bi[2];
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            sc[cs] = sc_next[cs];
            bi[cs] = bi_next[cs];
            // the next tile's factors, ahead of its epilogue (dropped past the
            // last tile)
            const uint32_t off =
                tile + 1 < t_end ? (uint32_t)(cur.co0 + (2 * cp + (hf_e == 0 ? cs : 1 - cs)) * 32 + l32_e) * 4u : kOOB;
            sc_next[cs] = __builtin_bit_cast(float, buf_load4(scr, off));
            bi_next[cs] = __builtin_bit_cast(float, buf_load4(bir, off));
        }
        static_for<0, NC>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int lb = m >> 1, cs = m & 1;
            const int pb = hf_e == 0 ? lb : PBX - 1 - lb;
            const int co = tb.co0 + (2 * cp + (hf_e == 0 ? cs : 1 - cs)) * 32 + l32_e;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int px = pb * 32 + 8 * q + 4 * hi_e;
                const int i = (int)(((uint32_t)px * rcp_tw) >> 20), j = px - i * tw_e;
                const int oh = tb.oh0 + i, ow = tb.ow0 + j;
                const bool ok = (px < tile_px) & (oh < s.OH) & (ow < s.OW) & (co < s.C_out);
                const float v0 = acc[m][4 * q], v1 = acc[m][4 * q + 1];
                const float v2 = acc[m][4 * q + 2], v3 = acc[m][4 * q + 3];
                u32x2 o;
                if (EPI == kFused) {
                    o.x = pack_bf16x2(bn_silu(v0, sc[cs], bi[cs]), bn_silu(v1, sc[cs], bi[cs]));
                    o.y = pack_bf16x2(bn_silu(v2, sc[cs], bi[cs]), bn_silu(v3, sc[cs], bi[cs]));
                } else {
                    o.x = pack_bf16x2(v0, v1);
                    o.y = pack_bf16x2(v2, v3);
                }
                buf_store8(yr, ok ? (uint32_t)(((tb.n * s.C_out + co) * s.OH + oh) * s.OW + ow) * 2u : kOOB, o);
            }
        });
    }
}

// Window geometry of a TH x TW tile; false if it does not fit.
bool make_geo32(const Shape &s, int TH, int TW, int vec, int num_cu, WinGeo *g) {
    g->TH = TH;
    g->TW = TW;
    g->FR = (TH - 1) * s.stride + s.KH;
    g->FC = (TW - 1) * s.stride + s.KW;
    g->CS = (g->FC + s.stride - 1) / s.stride;
    g->FCP = s.stride * g->CS;  // records a window row holds
    // Row pitch R >= FCP with S*R = TW (mod 16) (see the file comment).
    int R = g->FCP;
    while ((s.stride * R - TW) % 16 != 0) ++R;
    g->row_bytes = R * 16;
    if ((int64_t)2 * win_plane_bytes(g->FR, g->row_bytes) > kWinBytes) return false;
    g->ncg = (g->FC - 1 + vec - 1) / vec + 1;
    // the next chunk's window is staged by at most kTasks32 tasks per thread
    if (2 * g->FR * g->ncg > kMaxTasks32 * kThreads32) return false;
    g->tiles_h = (s.OH + TH - 1) / TH;
    g->tiles_w = (s.OW + TW - 1) / TW;
    g->co_tiles = (s.C_out + kBN32 - 1) / kBN32;
    g->n_tiles = s.N * g->tiles_h * g->tiles_w * g->co_tiles;
    g->n_chunks = (s.C_in + kCK32 - 1) / kCK32;
    g->n_chunks += g->n_chunks & 1;  // even: chunks run in pairs (a padding chunk adds zeros)
    g->tiles_per_wg = (g->n_tiles + num_cu - 1) / num_cu;
    g->n_wg = (g->n_tiles + g->tiles_per_wg - 1) / g->tiles_per_wg;
    return true;
}

constexpr int kTilePx = 13 * 32;  // pixels per tile, at most

// The tile (TW a multiple of 4, at most 416 pixels) that wastes the least
// matrix work: the share of the computed pixel slots (tiles x 416) that land
// on real output pixels, larger tiles on ties.  For a given TW only the
// tallest tile that fits is a candidate (a shorter one needs at least as
// many tiles), so planning costs a few dozen geometry checks.
bool plan32(const Shape &s, int vec, int num_cu, WinGeo *g) {
    int64_t best_tiles = 0, best_px = 0;
    WinGeo cand;
    for (int TW = 4; TW <= s.OW && TW <= kTilePx; TW += 4) {
        int TH = min(kTilePx / TW, s.OH);
        while (TH >= 1 && !make_geo32(s, TH, TW, vec, num_cu, &cand)) --TH;
        if (TH < 1) continue;
        const int64_t tiles = (int64_t)cand.tiles_h * cand.tiles_w;
        const int64_t px = (int64_t)TH * TW;
        if (best_tiles == 0 || tiles < best_tiles || (tiles == best_tiles && px > best_px)) {
            best_tiles = tiles;
            best_px = px;
            *g = cand;
        }
    }
    return best_tiles > 0;
}


}  // namespace

bool window32_supports(const Shape &s, int dtype) {
    if (dtype != kDtypeBf16 || s.W % 4 != 0 || s.OW % 4 != 0 || s.C_in % 8 != 0) return false;
    if (s.KH != 3 || s.KW != 3 || (s.stride != 1 && s.stride != 2)) return false;
    if ((uint64_t)s.N * s.C_in * s.HW * 2 > kMaxBufferBytes ||
        (uint64_t)s.N * s.C_out * s.OHW * 2 > kMaxBufferBytes || (uint64_t)s.C_out * s.K * 2 > kMaxBufferBytes)
        return false;
    WinGeo g;
    return plan32(s, kVec, 256, &g);
}

bool window32_pointers_ok(const void *x, const void *w, const void *y) {
    return (((uintptr_t)x | (uintptr_t)w) % 16 == 0) && (uintptr_t)y % 8 == 0;
}

// Share (per mille) of a tile's matrix work spent on real output pixels, for
// the dispatcher.
int window32_efficiency(const Shape &s) {
    WinGeo g;
    if (!plan32(s, kVec, 256, &g)) return 0;
    return (int)((int64_t)1000 * s.OH * s.OW / ((int64_t)g.tiles_h * g.tiles_w * kTilePx));
}

hipError_t launch_window32(const Shape &s, int epi, const void *x, const void *w, const float *scale,
                           const float *bias, void *y, hipStream_t st, int num_cu) {
    WinGeo g;
    if (!plan32(s, kVec, num_cu, &g)) return hipErrorInvalidValue;
    const int tasks = 2 * g.FR * g.ncg <= kThreads32 ? 1 : 2;
    const dim3 grid(g.n_wg), block(kThreads32);
    auto xx = (const uint16_t *)x;
    auto ww = (const uint16_t *)w;
    auto yy = (uint16_t *)y;
#define CBS_W32(S_, T_)                                                                                     \
    if (s.stride == S_ && tasks == T_) {                                                                    \
        if (epi == kFused)                                                                                  \
            hipLaunchKernelGGL((window32_bf16<S_, T_, kFused>), grid, block, 0, st, xx, ww, scale, bias, yy, \
                               s, g);                                                                      \
        else                                                                                                \
            hipLaunchKernelGGL((window32_bf16<S_, T_, kConvOnly>), grid, block, 0, st, xx, ww, scale, bias,  \
                               yy, s, g);                                                                  \
        return hipGetLastError();                                                                           \
    }
    CBS_W32(1, 1)
    CBS_W32(1, 2)
    CBS_W32(2, 1)
    CBS_W32(2, 2)
#undef CBS_W32
    return hipErrorInvalidValue;
}

}  // namespace cbs
