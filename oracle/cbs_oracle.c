/*
 * cbs_oracle.c -- CPU oracle for the fused conv2d + folded BatchNorm + SiLU
 * operator.  TEST INFRASTRUCTURE ONLY: nothing in the product path may link,
 * load or call this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.
 *
 * It computes the operator the slow, obvious way, in fp64, as the UNFUSED
 * three-operation sequence that "Fusing an Epilogue" (section "The problem")
 * contrasts with the fused kernel: the convolution produces an intermediate
 * t1 from x, batch norm turns t1 into a second intermediate t2, and SiLU
 * turns t2 into the output y, each step going through memory.
 *
 * Each pass is its own function with its own output array, so a reader can
 * check every step against the page by eye.  The page states that the fused
 * and unfused forms have identical arithmetic; the fused GPU kernel is checked
 * against this composition within a floating-point tolerance.
 *
 * Readings of points the page leaves open (each also listed in the design
 * notes of the repository):
 *   - "convolution" is cross-correlation (no kernel flip), zero padding, the
 *     same stride and padding on both spatial axes, dilation 1, one group;
 *   - x is NCHW [N][C_in][H][W], w is OIHW [C_out][C_in][KH][KW],
 *     t1/t2/y are NCHW [N][C_out][OH][OW] with OH = floor((H+2p-KH)/s)+1;
 *   - batch norm is the folded inference form, one scale and one shift per
 *     output channel: t2 = t1*scale[co] + bias[co] (order taken from the
 *     epilogue pseudocode in section "The shape of it");
 *   - sigmoid is the logistic function 1/(1+exp(-v)), and SiLU is v*sigmoid(v)
 *     (section "The problem").
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build.py).
 * -ffp-contract=off keeps every multiply and add separately rounded, so the
 * summation is exactly the loop order written below.
 *
 * Mutation hooks: when compiled with -DCBS_ORACLE_MUTANT=<k> (k > 0) the
 * oracle deliberately computes a WRONG result (a flipped kernel, a wrong pad
 * offset, a dropped bias, ...).  The CPU test suite builds these mutants and
 * checks that its pins reject every one of them.  The normal build defines
 * nothing and is the correct oracle.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>

#ifndef CBS_ORACLE_MUTANT
#define CBS_ORACLE_MUTANT 0
#endif

#define EXPORT __attribute__((visibility("default")))

/* Output spatial size, floor convention: OH = floor((H + 2p - KH)/s) + 1.
 * Returns -1 when the window does not fit (no output). */
EXPORT int cbs_oracle_out_dim(int in, int k, int stride, int pad)
{
    int span = in + 2 * pad - k;
#if CBS_ORACLE_MUTANT == 7
    span += 1; /* mutant: off-by-one in the output size */
#endif
    if (stride < 1 || span < 0)
        return -1;
    return span / stride + 1;
}

/* X(n, ci, ih, iw): the input with implicit zero padding outside [0,H)x[0,W). */
static double x_at(const double *x, int C_in, int H, int W,
                   int n, int ci, int ih, int iw)
{
    if (ih < 0 || ih >= H || iw < 0 || iw >= W)
        return 0.0;
    return x[(((size_t)n * C_in + ci) * H + ih) * W + iw];
}

/* Pass 1 -- convolution, x to t1.
 *   t1[n][co][oh][ow] = sum_{ci<C_in} sum_{kh<KH} sum_{kw<KW}
 *                       X(n, ci, oh*s - p + kh, ow*s - p + kw) * w[co][ci][kh][kw]
 * The sum runs in the fixed order ci, kh, kw.  OpenMP splits the (n, co)
 * planes over `nthreads` threads (0 = the OpenMP default); every output is
 * computed by exactly one thread, so the result does not depend on it.
 * Returns 0, or -1 for an invalid shape. */
EXPORT int cbs_oracle_conv(const double *x, const double *w, double *t1,
                           int N, int C_in, int H, int W, int C_out,
                           int KH, int KW, int stride, int pad, int nthreads)
{
    int OH = cbs_oracle_out_dim(H, KH, stride, pad);
    int OW = cbs_oracle_out_dim(W, KW, stride, pad);
    if (OH < 1 || OW < 1 || N < 0 || C_in < 1 || C_out < 1)
        return -1;
    long planes = (long)N * C_out;
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long pl = 0; pl < planes; ++pl) {
        int n = (int)(pl / C_out);
        int co = (int)(pl % C_out);
        double *out = t1 + (size_t)pl * OH * OW;
        for (int oh = 0; oh < OH; ++oh) {
            for (int ow = 0; ow < OW; ++ow) {
                double acc = 0.0;
                for (int ci = 0; ci < C_in; ++ci) {
                    for (int kh = 0; kh < KH; ++kh) {
                        for (int kw = 0; kw < KW; ++kw) {
#if CBS_ORACLE_MUTANT == 1
                            /* mutant: true convolution (flipped kernel) */
                            double wv = w[(((size_t)co * C_in + ci) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)];
#elif CBS_ORACLE_MUTANT == 5
                            /* mutant: kh and kw swapped in the weight index */
                            double wv = w[(((size_t)co * C_in + ci) * KH + kw % KH) * KW + kh % KW];
#else
                            double wv = w[(((size_t)co * C_in + ci) * KH + kh) * KW + kw];
#endif
#if CBS_ORACLE_MUTANT == 2
                            /* mutant: padding applied with the wrong sign */
                            int ih = oh * stride + pad + kh;
#else
                            int ih = oh * stride - pad + kh;
#endif
                            int iw = ow * stride - pad + kw;
#if CBS_ORACLE_MUTANT == 6
                            /* mutant: the last input channel is dropped */
                            if (ci == C_in - 1 && C_in > 1)
                                continue;
#endif
                            acc += x_at(x, C_in, H, W, n, ci, ih, iw) * wv;
                        }
                    }
                }
                out[(size_t)oh * OW + ow] = acc;
            }
        }
    }
    return 0;
}

/* Pass 2 -- folded batch norm, t1 to t2: each element scaled and shifted by
 * the parameters of its output channel:
 *   t2[n][co][i] = t1[n][co][i] * scale[co] + bias[co]. */
EXPORT void cbs_oracle_bn(const double *t1, const double *scale, const double *bias,
                          double *t2, int N, int C_out, long plane)
{
    long planes = (long)N * C_out;
#pragma omp parallel for schedule(static)
    for (long pl = 0; pl < planes; ++pl) {
        int co = (int)(pl % C_out);
        const double *src = t1 + (size_t)pl * plane;
        double *dst = t2 + (size_t)pl * plane;
        for (long i = 0; i < plane; ++i) {
#if CBS_ORACLE_MUTANT == 3
            dst[i] = src[i] * scale[co]; /* mutant: bias dropped */
#else
            dst[i] = src[i] * scale[co] + bias[co];
#endif
        }
    }
}

/* The logistic function 1/(1+exp(-v)). */
static double sigmoid(double v)
{
#if CBS_ORACLE_MUTANT == 4
    return 1.0 / (1.0 + exp(v)); /* mutant: wrong sign in the exponent */
#else
    return 1.0 / (1.0 + exp(-v));
#endif
}

/* Pass 3 -- SiLU, t2 to y: y = v * sigmoid(v).
 * For v below about -709, exp(-v) overflows to +inf, sigmoid(v) = 0 and
 * y = -0.0, which is the correctly rounded limit. */
EXPORT void cbs_oracle_silu(const double *t2, double *y, long count)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < count; ++i)
        y[i] = t2[i] * sigmoid(t2[i]);
}

/* The three passes in sequence, into caller-provided t1, t2 and y. */
EXPORT int cbs_oracle_forward(const double *x, const double *w,
                              const double *scale, const double *bias,
                              double *t1, double *t2, double *y,
                              int N, int C_in, int H, int W, int C_out,
                              int KH, int KW, int stride, int pad, int nthreads)
{
    int rc = cbs_oracle_conv(x, w, t1, N, C_in, H, W, C_out, KH, KW, stride, pad, nthreads);
    if (rc != 0)
        return rc;
    int OH = cbs_oracle_out_dim(H, KH, stride, pad);
    int OW = cbs_oracle_out_dim(W, KW, stride, pad);
    long plane = (long)OH * OW;
    cbs_oracle_bn(t1, scale, bias, t2, N, C_out, plane);
    cbs_oracle_silu(t2, y, (long)N * C_out * plane);
    return 0;
}

/* Sampled outputs for workloads too large to run whole: for each flat NCHW
 * output index idx[i] (into [N][C_out][OH][OW]) the three steps are taken
 * for that one element -- the conv sum in the order ci, kh, kw, then the
 * multiply-add of its channel, then SiLU -- and written to y[i].
 * Returns 0, or -1 for an invalid shape or index. */
EXPORT int cbs_oracle_points(const double *x, const double *w,
                             const double *scale, const double *bias,
                             const int64_t *idx, long count, double *y,
                             int N, int C_in, int H, int W, int C_out,
                             int KH, int KW, int stride, int pad)
{
    int OH = cbs_oracle_out_dim(H, KH, stride, pad);
    int OW = cbs_oracle_out_dim(W, KW, stride, pad);
    if (OH < 1 || OW < 1)
        return -1;
    int64_t total = (int64_t)N * C_out * OH * OW;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (long i = 0; i < count; ++i) {
        int64_t m = idx[i];
        if (m < 0 || m >= total) {
            bad = 1;
            continue;
        }
        int ow = (int)(m % OW);
        int oh = (int)((m / OW) % OH);
        int co = (int)((m / ((int64_t)OW * OH)) % C_out);
        int n = (int)(m / ((int64_t)OW * OH * C_out));
        double acc = 0.0;
        for (int ci = 0; ci < C_in; ++ci)
            for (int kh = 0; kh < KH; ++kh)
                for (int kw = 0; kw < KW; ++kw)
                    acc += x_at(x, C_in, H, W, n, ci, oh * stride - pad + kh, ow * stride - pad + kw) *
                           w[(((size_t)co * C_in + ci) * KH + kh) * KW + kw];
        double t2 = acc * scale[co] + bias[co];
        y[i] = t2 * sigmoid(t2);
    }
    return bad ? -1 : 0;
}
