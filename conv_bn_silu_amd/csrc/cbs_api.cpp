// cbs_api.cpp -- the C ABI declared in include/conv_bn_silu.h: handles,
// host-side validation, variant dispatch and kernel launch.
//
// Nothing here touches device memory and nothing allocates it: every
// argument is checked before the first HIP call, every failure is reported as
// a status code, and a run call only enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <set>

#include "../../include/conv_bn_silu.h"
#include "cbs_launch.h"
#include "cbs_shape.h"

struct conv_bn_silu_handle {
    // Fixed at create and only read afterwards, so one handle may serve
    // concurrent calls from any number of threads and streams.
    int device;
    int num_cu;
    // Device address of the allocation-free entry point's scratch on this
    // device (NULL if the lookup failed; that entry point then reports it).
    void *noalloc_scratch;
};

namespace {

std::mutex g_handles_mu;
std::set<const conv_bn_silu_handle *> g_handles;  // live handles; never dereference a foreign pointer

// The hipError_t of the last failed HIP call this thread made through the
// library (kept per thread, so that handles stay read-only).
thread_local int t_last_hip_error = 0;

bool handle_live(const conv_bn_silu_handle *h) {
    std::lock_guard<std::mutex> lk(g_handles_mu);
    return h != nullptr && g_handles.count(h) != 0;
}

// Geometry and overflow checks; fills `s` on success.
int check_shape(int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
                int dtype, cbs::Shape *s) {
    if (dtype != CBS_DTYPE_F32 && dtype != CBS_DTYPE_BF16) return CBS_ERR_INVALID_ARG;
    if (N < 0 || C_in < 1 || H < 1 || W < 1 || C_out < 1 || KH < 1 || KW < 1 || stride < 1 || pad < 0)
        return CBS_ERR_INVALID_ARG;
    const int64_t span_h = (int64_t)H + 2 * (int64_t)pad - KH;
    const int64_t span_w = (int64_t)W + 2 * (int64_t)pad - KW;
    if (span_h < 0 || span_w < 0) return CBS_ERR_INVALID_ARG;  // the window does not fit
    const int64_t OH = span_h / stride + 1, OW = span_w / stride + 1;
    const int64_t lim = INT32_MAX;
    const int64_t x_el = (int64_t)N * C_in * H * W;
    const int64_t w_el = (int64_t)C_out * C_in * KH * KW;
    const int64_t y_el = (int64_t)N * C_out * OH * OW;
    // 32-bit index arithmetic inside the kernels must be exact, including the
    // padded coordinates oh*stride - pad + kh.
    if (x_el > lim || w_el > lim || y_el > lim || (int64_t)H + 2 * (int64_t)pad > lim ||
        (int64_t)W + 2 * (int64_t)pad > lim || (int64_t)H * W > lim || (int64_t)N * OH * OW > lim)
        return CBS_ERR_UNSUPPORTED;
    s->N = N; s->C_in = C_in; s->H = H; s->W = W; s->C_out = C_out;
    s->KH = KH; s->KW = KW; s->stride = stride; s->pad = pad;
    s->OH = (int)OH; s->OW = (int)OW;
    s->M = (int)(N * OH * OW);
    s->K = C_in * KH * KW;
    s->HW = H * W;
    s->OHW = (int)(OH * OW);
    s->T = KH * KW;
    return CBS_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_pointers(const void *x, const void *w, const float *scale, const float *bias, const void *y,
                   const cbs::Shape &s, int dtype) {
    if (!x || !w || !scale || !bias || !y) return CBS_ERR_INVALID_ARG;
    const uintptr_t e = dtype == CBS_DTYPE_BF16 ? 2 : 4;
    const Range rx{(uintptr_t)x, (uintptr_t)x + (uintptr_t)s.N * s.C_in * s.HW * e};
    const Range rw{(uintptr_t)w, (uintptr_t)w + (uintptr_t)s.C_out * s.K * e};
    const Range rs{(uintptr_t)scale, (uintptr_t)scale + (uintptr_t)s.C_out * 4};
    const Range rb{(uintptr_t)bias, (uintptr_t)bias + (uintptr_t)s.C_out * 4};
    const Range ry{(uintptr_t)y, (uintptr_t)y + (uintptr_t)s.N * s.C_out * s.OHW * e};
    if (overlap(ry, rx) || overlap(ry, rw) || overlap(ry, rs) || overlap(ry, rb)) return CBS_ERR_INVALID_ARG;
    // Pointers off their element size are well-formed requests the kernels
    // do not serve.
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) % e != 0) return CBS_ERR_UNSUPPORTED;
    if (((uintptr_t)scale | (uintptr_t)bias) % 4 != 0) return CBS_ERR_UNSUPPORTED;
    return CBS_OK;
}

int validate_all(const void *x, const void *w, const float *scale, const float *bias, const void *y, int N,
                 int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad, int dtype,
                 cbs::Shape *s) {
    const int rc = check_shape(N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, s);
    if (rc != CBS_OK) return rc;
    if (N == 0) return CBS_OK;  // nothing to do; pointers are not looked at
    return check_pointers(x, w, scale, bias, y, *s, dtype);
}

bool variant_ok(int variant, const cbs::Shape &s, int dtype) {
    switch (variant) {
        case CBS_VARIANT_GEMM_GATHER: return cbs::gemm_gather_supports(s, dtype);
        case CBS_VARIANT_GEMM_WINDOW: return cbs::window_supports(s, dtype);
        case CBS_VARIANT_GEMM_WINDOW32: return cbs::window32_supports(s, dtype);
        case CBS_VARIANT_POINTWISE: return cbs::pointwise_supports(s, dtype);
        case CBS_VARIANT_SMALL_K: return cbs::stem_supports(s, dtype);
        case CBS_VARIANT_ROWS: return cbs::rows_supports(s, dtype);
        case CBS_VARIANT_SCALAR: return cbs::scalar_supports(s, dtype);
        default: return false;
    }
}

// Alignment the vectorised variants need beyond element alignment.
bool pointers_ok(int variant, const void *x, const void *w, const void *y) {
    switch (variant) {
        case CBS_VARIANT_POINTWISE: return cbs::pointwise_pointers_ok(x, w, y);
        case CBS_VARIANT_SMALL_K: return cbs::stem_pointers_ok(x, w, y);
        case CBS_VARIANT_ROWS: return cbs::rows_pointers_ok(x, w, y);
        case CBS_VARIANT_GEMM_WINDOW: return cbs::window_pointers_ok(x, w, y);
        case CBS_VARIANT_GEMM_WINDOW32: return cbs::window32_pointers_ok(x, w, y);
        default: return true;
    }
}

// AUTO dispatch.  Shape rules in the spirit of the page's hand-picked
// thresholds ("Three kernels for one operation"), set here from measurement
// on MI355X (bench.py --variants times every variant on shapes on both sides
// of each rule): the scalar kernel for problems too small for any tiling to
// pay (up to 2^24 multiply-adds in bf16; in fp32, where the tiled kernel runs
// on the slower fp32 matrix instructions, up to 2^27), then the specialised
// kernels where the shape fits them, the 32x32 window kernel for any 3x3
// layer it serves, the 16x16 window kernel for other filters larger than
// 1x1, and the generic implicit GEMM otherwise.
int select(const cbs::Shape &s, int dtype, int num_cu) {
    (void)num_cu;  // the rules are measured on 256 compute units; tiling already adapts to the count
    const int64_t macs = (int64_t)s.M * s.C_out * s.K;
    const int64_t scalar_limit = dtype == CBS_DTYPE_F32 ? (int64_t)1 << 27 : (int64_t)1 << 24;
    if (macs <= scalar_limit && variant_ok(CBS_VARIANT_SCALAR, s, dtype)) return CBS_VARIANT_SCALAR;
    if (variant_ok(CBS_VARIANT_POINTWISE, s, dtype)) return CBS_VARIANT_POINTWISE;
    if (variant_ok(CBS_VARIANT_SMALL_K, s, dtype)) return CBS_VARIANT_SMALL_K;
    if (variant_ok(CBS_VARIANT_ROWS, s, dtype)) return CBS_VARIANT_ROWS;
    if (variant_ok(CBS_VARIANT_GEMM_WINDOW32, s, dtype)) return CBS_VARIANT_GEMM_WINDOW32;
    if (s.T > 1 && variant_ok(CBS_VARIANT_GEMM_WINDOW, s, dtype)) return CBS_VARIANT_GEMM_WINDOW;
    return CBS_VARIANT_GEMM_GATHER;
}

// AUTO dispatch at run time: the shape's choice, unless its pointers are not
// aligned for it, in which case the generic kernel serves the call.
int select_for_call(const cbs::Shape &s, int dtype, int num_cu, const void *x, const void *w, const void *y) {
    const int v = select(s, dtype, num_cu);
    return pointers_ok(v, x, w, y) ? v : CBS_VARIANT_GEMM_GATHER;
}

hipError_t launch(int variant, const cbs::Shape &s, int dtype, int epi, const void *x, const void *w,
                  const float *scale, const float *bias, void *y, hipStream_t st, int num_cu) {
    // hipGetLastError reports the last error of any HIP call on this thread;
    // clear whatever an earlier, unrelated call left so that the launcher's
    // check sees only its own launch.
    (void)hipGetLastError();
    switch (variant) {
        case CBS_VARIANT_GEMM_GATHER: return cbs::launch_gemm_gather(s, dtype, epi, x, w, scale, bias, y, st);
        case CBS_VARIANT_POINTWISE: return cbs::launch_pointwise(s, epi, x, w, scale, bias, y, st, num_cu);
        case CBS_VARIANT_GEMM_WINDOW:
            return cbs::launch_window(s, epi, x, w, scale, bias, y, st, num_cu);
        case CBS_VARIANT_GEMM_WINDOW32:
            return cbs::launch_window32(s, epi, x, w, scale, bias, y, st, num_cu);
        case CBS_VARIANT_SMALL_K: return cbs::launch_stem(s, epi, x, w, scale, bias, y, st, num_cu);
        case CBS_VARIANT_ROWS: return cbs::launch_rows(s, epi, x, w, scale, bias, y, st, num_cu);
        case CBS_VARIANT_SCALAR: return cbs::launch_scalar(s, dtype, epi, x, w, scale, bias, y, st);
        default: return hipErrorInvalidValue;
    }
}

int record_hip(hipError_t e) {
    if (e == hipSuccess) return CBS_OK;
    t_last_hip_error = (int)e;
    return CBS_ERR_HIP;
}

// Common front half of the run entry points: handle, arguments, device.
int prologue(conv_bn_silu_t h, const void *x, const void *w, const float *scale, const float *bias,
             const void *y, int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
             int dtype, cbs::Shape *s) {
    if (!handle_live(h)) return CBS_ERR_BAD_HANDLE;
    const int rc = validate_all(x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, s);
    if (rc != CBS_OK) return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CBS_ERR_NO_DEVICE;
    if (dev != h->device) return CBS_ERR_INVALID_ARG;  // the handle belongs to another device
    return CBS_OK;
}

// The unfused sequence on t1, t2 (validated by the caller): the AUTO
// variant's convolution without its epilogue, then the BN pass, then SiLU.
int launch_unfused(const conv_bn_silu_handle *h, const cbs::Shape &s, int dtype, const void *x, const void *w,
                   const float *scale, const float *bias, void *t1, void *t2, void *y, hipStream_t st) {
    const int variant = select_for_call(s, dtype, h->num_cu, x, w, t1);
    int rc = record_hip(launch(variant, s, dtype, cbs::kConvOnly, x, w, scale, bias, t1, st, h->num_cu));
    if (rc != CBS_OK) return rc;
    (void)hipGetLastError();
    rc = record_hip(cbs::launch_bn_pass(s, dtype, t1, scale, bias, t2, st));
    if (rc != CBS_OK) return rc;
    (void)hipGetLastError();
    return record_hip(cbs::launch_silu_pass(s, dtype, t2, y, st));
}

}  // namespace

extern "C" {

int conv_bn_silu_create(conv_bn_silu_t *out_handle) {
    if (!out_handle) return CBS_ERR_INVALID_ARG;
    *out_handle = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) return CBS_ERR_NO_DEVICE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CBS_ERR_NO_DEVICE;
    // Scalar attributes only (no property record, whose layout depends on the
    // runtime release).  The graphics IP version of gfx950 is 9.5.
    int major = 0, minor = 0, num_cu = 0;
    if (hipDeviceGetAttribute(&major, hipDeviceAttributeComputeCapabilityMajor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&minor, hipDeviceAttributeComputeCapabilityMinor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return CBS_ERR_NO_DEVICE;
    if (major != 9 || minor != 5 || num_cu < 1) return CBS_ERR_UNSUPPORTED;
    auto *h = new conv_bn_silu_handle;
    h->device = dev;
    h->num_cu = num_cu;
    h->noalloc_scratch = nullptr;
    if (cbs::noalloc_scratch_address(&h->noalloc_scratch) != hipSuccess) h->noalloc_scratch = nullptr;
    (void)hipGetLastError();
    {
        std::lock_guard<std::mutex> lk(g_handles_mu);
        g_handles.insert(h);
    }
    *out_handle = h;
    return CBS_OK;
}

int conv_bn_silu_destroy(conv_bn_silu_t h) {
    if (!h) return CBS_OK;
    {
        std::lock_guard<std::mutex> lk(g_handles_mu);
        if (g_handles.erase(h) == 0) return CBS_ERR_BAD_HANDLE;
    }
    delete h;
    return CBS_OK;
}

int conv_bn_silu_run_variant(conv_bn_silu_t h, int variant, const void *x, const void *w, const float *scale,
                             const float *bias, void *y, int N, int C_in, int H, int W, int C_out, int KH, int KW,
                             int stride, int pad, int dtype, void *stream) {
    if (variant < 0 || variant >= CBS_VARIANT_COUNT_) return CBS_ERR_INVALID_ARG;
    cbs::Shape s;
    int rc = prologue(h, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s);
    if (rc != CBS_OK) return rc;
    if (s.N == 0) return CBS_OK;
    if (variant == CBS_VARIANT_AUTO) variant = select_for_call(s, dtype, h->num_cu, x, w, y);
    else if (!variant_ok(variant, s, dtype) || !pointers_ok(variant, x, w, y)) return CBS_ERR_UNSUPPORTED;
    return record_hip(launch(variant, s, dtype, cbs::kFused, x, w, scale, bias, y, (hipStream_t)stream,
                             h->num_cu));
}

int conv_bn_silu_run(conv_bn_silu_t h, const void *x, const void *w, const float *scale, const float *bias,
                     void *y, int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
                     int dtype, void *stream) {
    return conv_bn_silu_run_variant(h, CBS_VARIANT_AUTO, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW,
                                    stride, pad, dtype, stream);
}

int conv_bn_silu_run_unfused(conv_bn_silu_t h, const void *x, const void *w, const float *scale,
                             const float *bias, void *t1, void *t2, void *y, int N, int C_in, int H, int W,
                             int C_out, int KH, int KW, int stride, int pad, int dtype, void *stream) {
    cbs::Shape s;
    int rc = prologue(h, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s);
    if (rc != CBS_OK) return rc;
    if (s.N == 0) return CBS_OK;
    const uintptr_t e = dtype == CBS_DTYPE_BF16 ? 2 : 4;
    if (!t1 || !t2) return CBS_ERR_INVALID_ARG;
    const uintptr_t ybytes = (uintptr_t)s.N * s.C_out * s.OHW * e;
    const Range r1{(uintptr_t)t1, (uintptr_t)t1 + ybytes}, r2{(uintptr_t)t2, (uintptr_t)t2 + ybytes};
    const Range others[] = {{(uintptr_t)x, (uintptr_t)x + (uintptr_t)s.N * s.C_in * s.HW * e},
                            {(uintptr_t)w, (uintptr_t)w + (uintptr_t)s.C_out * s.K * e},
                            {(uintptr_t)scale, (uintptr_t)scale + (uintptr_t)s.C_out * 4},
                            {(uintptr_t)bias, (uintptr_t)bias + (uintptr_t)s.C_out * 4},
                            {(uintptr_t)y, (uintptr_t)y + ybytes}};
    if (overlap(r1, r2)) return CBS_ERR_INVALID_ARG;
    for (const Range &o : others)
        if (overlap(r1, o) || overlap(r2, o)) return CBS_ERR_INVALID_ARG;
    if (((uintptr_t)t1 | (uintptr_t)t2) % e != 0) return CBS_ERR_UNSUPPORTED;
    return launch_unfused(h, s, dtype, x, w, scale, bias, t1, t2, y, (hipStream_t)stream);
}

int conv_bn_silu_run_unfused_noalloc(conv_bn_silu_t h, const void *x, const void *w, const float *scale,
                                     const float *bias, void *y, int N, int C_in, int H, int W, int C_out, int KH,
                                     int KW, int stride, int pad, int dtype, void *stream) {
    cbs::Shape s;
    const int rc = prologue(h, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s);
    if (rc != CBS_OK) return rc;
    if (s.N == 0) return CBS_OK;
    const uint64_t half = cbs::kNoAllocScratchBytes / 2;
    const uint64_t ybytes = (uint64_t)s.N * s.C_out * s.OHW * (dtype == CBS_DTYPE_BF16 ? 2 : 4);
    if (ybytes > half) return CBS_ERR_UNSUPPORTED;  // an intermediate does not fit its half of the scratch
    if (!h->noalloc_scratch) return record_hip(hipErrorInvalidSymbol);
    void *t1 = h->noalloc_scratch;
    void *t2 = (unsigned char *)h->noalloc_scratch + half;
    return launch_unfused(h, s, dtype, x, w, scale, bias, t1, t2, y, (hipStream_t)stream);
}

int conv_bn_silu_output_hw(int H, int W, int KH, int KW, int stride, int pad, int *OH, int *OW) {
    if (!OH || !OW) return CBS_ERR_INVALID_ARG;
    cbs::Shape s;
    const int rc = check_shape(1, 1, H, W, 1, KH, KW, stride, pad, CBS_DTYPE_F32, &s);
    if (rc != CBS_OK) return rc;
    *OH = s.OH;
    *OW = s.OW;
    return CBS_OK;
}

int conv_bn_silu_validate(const void *x, const void *w, const float *scale, const float *bias, const void *y,
                          int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
                          int dtype) {
    cbs::Shape s;
    return validate_all(x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s);
}

int conv_bn_silu_select_variant(int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
                                int dtype, int num_cu) {
    cbs::Shape s;
    if (check_shape(N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s) != CBS_OK) return -1;
    return select(s, dtype, num_cu);
}

int conv_bn_silu_variant_supports(int variant, int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                  int stride, int pad, int dtype) {
    cbs::Shape s;
    if (check_shape(N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, &s) != CBS_OK) return 0;
    if (variant == CBS_VARIANT_AUTO) return 1;
    return variant_ok(variant, s, dtype) ? 1 : 0;
}

const char *conv_bn_silu_status_string(int status) {
    switch (status) {
        case CBS_OK: return "ok";
        case CBS_ERR_INVALID_ARG: return "invalid argument";
        case CBS_ERR_UNSUPPORTED: return "unsupported (device, size or variant)";
        case CBS_ERR_NO_DEVICE: return "no HIP device";
        case CBS_ERR_HIP: return "HIP runtime error";
        case CBS_ERR_BAD_HANDLE: return "bad handle";
        default: return "unknown";
    }
}

const char *conv_bn_silu_variant_name(int variant) {
    switch (variant) {
        case CBS_VARIANT_AUTO: return "auto";
        case CBS_VARIANT_GEMM_GATHER: return "gemm_gather";
        case CBS_VARIANT_GEMM_WINDOW: return "gemm_window";
        case CBS_VARIANT_POINTWISE: return "pointwise";
        case CBS_VARIANT_SMALL_K: return "small_k";
        case CBS_VARIANT_SCALAR: return "scalar";
        case CBS_VARIANT_GEMM_WINDOW32: return "gemm_window32";
        case CBS_VARIANT_ROWS: return "strided_rows";
        default: return "unknown";
    }
}

int conv_bn_silu_last_hip_error(conv_bn_silu_t h) {
    if (!handle_live(h)) return 0;
    return t_last_hip_error;
}

int conv_bn_silu_fold_bn(const float *gamma, const float *beta, const float *mean, const float *var, float eps,
                         const float *conv_bias, int C_out, float *scale, float *bias) {
    if (!gamma || !beta || !mean || !var || !scale || !bias || C_out < 1 || !(eps >= 0.f))
        return CBS_ERR_INVALID_ARG;
    for (int c = 0; c < C_out; ++c)
        if (!((double)var[c] + (double)eps > 0.0)) return CBS_ERR_INVALID_ARG;
    for (int c = 0; c < C_out; ++c) {
        const double sc = (double)gamma[c] / std::sqrt((double)var[c] + (double)eps);
        const double cb = conv_bias ? (double)conv_bias[c] : 0.0;
        scale[c] = (float)sc;
        bias[c] = (float)((double)beta[c] + (cb - (double)mean[c]) * sc);
    }
    return CBS_OK;
}

}  // extern "C"
