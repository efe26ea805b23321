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

// Epilogue modes: the fused operator, or the plain convolution (the first
// kernel of the unfused sequence).
enum Epilogue { kFused = 0, kConvOnly = 1 };

}  // namespace cbs
