// cbs_shape.h -- geometry of one convolution call, shared by the host library
// and the kernels (plain C++, no HIP types).
#pragma once

#include <stdint.h>

namespace cbs {

// One call's geometry.  Implicit-GEMM view: M = N*OH*OW output pixels (rows),
// C_out output channels (columns), K = C_in*KH*KW reduction length, with
// k = (ci*KH + kh)*KW + kw (the OIHW order of w) unless a kernel says
// otherwise.  Every tensor holds fewer than 2^31 elements, so 32-bit indexing
// is exact.
struct Shape {
    int N, C_in, H, W, C_out, KH, KW, stride, pad;
    int OH, OW;
    int M;    // N * OH * OW
    int K;    // C_in * KH * KW
    int HW;   // H * W
    int OHW;  // OH * OW
    int T;    // KH * KW (kernel taps)
};

// Tiling of the window kernel: TH x TW output pixels per tile; the input
// window of a tile is FR rows x FC columns, stored with row pitch FCP
// records and, for stride > 1, columns grouped by residue (CS per group).
struct WinGeo {
    int TH, TW, FR, FC, CS, FCP;
    int row_bytes;                     // LDS bytes per window row (32-channel records)
    int ncg;                           // staging column groups per window row
    int tiles_h, tiles_w, co_tiles, n_tiles;
    int n_chunks;                      // 32-channel blocks of C_in
    int tiles_per_wg, n_wg;            // contiguous tile run per workgroup, workgroups
};

// Epilogue modes: the fused operator, or the plain convolution (the first
// kernel of the unfused sequence).
enum Epilogue { kFused = 0, kConvOnly = 1 };

}  // namespace cbs
