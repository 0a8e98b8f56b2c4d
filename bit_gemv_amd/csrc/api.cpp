// api.cpp -- the extern "C" entry points of libquant (declared in
// include/libquant.h): argument validation, then one launch on the caller's
// stream. No allocation, no host<->device copies, no synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/libquant.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

lq_status fail(lq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

// Device presence, checked once per process after a first success.
std::atomic<int> g_have_device{0};

lq_status need_device() {
    if (g_have_device.load(std::memory_order_relaxed)) return LQ_OK;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(LQ_ERR_NO_DEVICE, "no HIP device visible (%s)", hipGetErrorString(e));
    }
    g_have_device.store(1, std::memory_order_relaxed);
    return LQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    const void *p;
    int64_t bytes;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Every output range must be disjoint from every input range and from the
// other outputs.
bool any_overlap(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range &i : ins)
            if (overlap(*o, i)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return true;
    }
    return false;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// largest multiple of 128 with k * 128 * 128 < 2^31 (W8A8 int32 accumulators)
constexpr int64_t kMaxW8a8K = 130944;

lq_status launched(hipError_t e, const char *what) {
    if (e == hipErrorNotSupported) return fail(LQ_ERR_UNSUPPORTED, "%s: not available in this build", what);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    }
    g_err[0] = '\0';
    return LQ_OK;
}

// Shared checks of the (bits, group, k) triple for quantize/dequantize.
lq_status check_group(const char *fn, int64_t k, int bits, int64_t group) {
    if (bits != 4 && bits != 8) return fail(LQ_ERR_INVALID_ARG, "%s: bits must be 4 or 8 (got %d)", fn, bits);
    if (k <= 0 || group <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: k and group must be positive", fn);
    if (k % group != 0) return fail(LQ_ERR_INVALID_ARG, "%s: k (%lld) is not a multiple of group (%lld)", fn,
                                    (long long)k, (long long)group);
    if (group % 128 != 0)
        return fail(LQ_ERR_UNSUPPORTED, "%s: group must be a multiple of 128 (got %lld)", fn, (long long)group);
    if (k > kMaxDim) return fail(LQ_ERR_UNSUPPORTED, "%s: k too large", fn);
    return LQ_OK;
}

lq_status check_meta(const char *fn, int symmetric, const float *scales, const float *zeros) {
    if (!scales || !aligned(scales, 4)) return fail(LQ_ERR_INVALID_ARG, "%s: scales null or misaligned", fn);
    if (symmetric && zeros) return fail(LQ_ERR_INVALID_ARG, "%s: zeros must be NULL for symmetric", fn);
    if (!symmetric && (!zeros || !aligned(zeros, 4)))
        return fail(LQ_ERR_INVALID_ARG, "%s: zeros null or misaligned for asymmetric", fn);
    return LQ_OK;
}

// Arguments of the weight-only products (INT4 or INT8 codes, bf16 x).
lq_status check_wo(const char *fn, int bits, const void *x, int64_t m, const void *codes, const float *scales,
                   const float *zeros, int64_t n, int64_t k, int symmetric, int64_t group, const float *y) {
    if (m < 0 || n < 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative size", fn);
    lq_status st = check_group(fn, k, bits, group);
    if (st != LQ_OK) return st;
    if (n > kMaxDim || m > kMaxDim) return fail(LQ_ERR_UNSUPPORTED, "%s: dimension too large", fn);
    // kernels address a few rows of codes with 32-bit buffer offsets
    if (k > (int64_t(1) << 28)) return fail(LQ_ERR_UNSUPPORTED, "%s: k > 2^28", fn);
    if (m == 0 || n == 0) return LQ_OK;
    if (!x || !aligned(x, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (!y || !aligned(y, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: y null or not 16-byte aligned", fn);
    st = check_meta(fn, symmetric, scales, zeros);
    if (st != LQ_OK) return st;
    const int64_t meta = n * (k / group) * 4;
    if (any_overlap({{y, m * n * 4}},
                    {{x, m * k * 2}, {codes, bits == 4 ? n * k / 2 : n * k}, {scales, meta},
                     {zeros, symmetric ? 0 : meta}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    return LQ_OK;
}

}  // namespace

extern "C" {

int lq_abi_version(void) { return LQ_ABI_VERSION; }

const char *lq_status_string(lq_status s) {
    switch (s) {
        case LQ_OK: return "ok";
        case LQ_ERR_INVALID_ARG: return "invalid argument";
        case LQ_ERR_UNSUPPORTED: return "unsupported";
        case LQ_ERR_HIP: return "HIP error";
        case LQ_ERR_NO_DEVICE: return "no device";
    }
    return "unknown status";
}

const char *lq_last_error(void) { return g_err; }

lq_status quantize_groupwise(const void *w_bf16, int64_t n, int64_t k, int bits, int symmetric, int64_t group,
                             const float *col_scale, void *codes, float *scales, float *zeros, void *stream) {
    const char *fn = "quantize_groupwise";
    if (n < 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative n", fn);
    lq_status st = check_group(fn, k, bits, group);
    if (st != LQ_OK) return st;
    if (n > kMaxDim || n * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: matrix too large", fn);
    if (n == 0) return LQ_OK;
    if (!w_bf16 || !aligned(w_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: w null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (col_scale && !aligned(col_scale, 16))
        return fail(LQ_ERR_INVALID_ARG, "%s: col_scale not 16-byte aligned", fn);
    st = check_meta(fn, symmetric, scales, zeros);
    if (st != LQ_OK) return st;
    const int64_t meta = n * (k / group) * 4;
    const int64_t cbytes = bits == 4 ? n * k / 2 : n * k;
    if (any_overlap({{codes, cbytes}, {scales, meta}, {zeros, symmetric ? 0 : meta}},
                    {{w_bf16, n * k * 2}, {col_scale, col_scale ? k * 4 : 0}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output overlaps an input or another output", fn);
    if ((st = need_device()) != LQ_OK) return st;
    lq::QuantArgs a{static_cast<const uint16_t *>(w_bf16), n, k, bits, symmetric, group, col_scale,
                    static_cast<uint8_t *>(codes), scales, zeros};
    return launched(lq::launch_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status dequantize_groupwise(const void *codes, const float *scales, const float *zeros, int64_t n, int64_t k,
                               int bits, int symmetric, int64_t group, float *out, void *stream) {
    const char *fn = "dequantize_groupwise";
    if (n < 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative n", fn);
    lq_status st = check_group(fn, k, bits, group);
    if (st != LQ_OK) return st;
    if (n > kMaxDim || n * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: matrix too large", fn);
    if (n == 0) return LQ_OK;
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (!out || !aligned(out, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: out null or not 16-byte aligned", fn);
    st = check_meta(fn, symmetric, scales, zeros);
    if (st != LQ_OK) return st;
    const int64_t meta = n * (k / group) * 4;
    const int64_t cbytes = bits == 4 ? n * k / 2 : n * k;
    if (any_overlap({{out, n * k * 4}}, {{codes, cbytes}, {scales, meta}, {zeros, symmetric ? 0 : meta}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    if ((st = need_device()) != LQ_OK) return st;
    lq::DequantArgs a{static_cast<const uint8_t *>(codes), scales, zeros, n, k, bits, symmetric, group, out};
    return launched(lq::launch_dequantize(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status w4a16_gemv(const void *x_bf16, int64_t b, const void *codes, const float *scales, const float *zeros,
                     int64_t n, int64_t k, int symmetric, int64_t group, float *y, void *stream) {
    const char *fn = "w4a16_gemv";
    if (b > 16) return fail(LQ_ERR_UNSUPPORTED, "%s: batch %lld > 16 (use w4a16_gemm)", fn, (long long)b);
    lq_status st = check_wo(fn, 4, x_bf16, b, codes, scales, zeros, n, k, symmetric, group, y);
    if (st != LQ_OK || b == 0 || n == 0) return st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::WoArgs a{static_cast<const uint16_t *>(x_bf16), b, static_cast<const uint8_t *>(codes), scales, zeros,
                 n, k, symmetric, group, y};
    return launched(lq::launch_w4a16_gemv(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status w8a16_gemv(const void *x_bf16, int64_t b, const void *codes, const float *scales, const float *zeros,
                     int64_t n, int64_t k, int symmetric, int64_t group, float *y, void *stream) {
    const char *fn = "w8a16_gemv";
    if (b > 16) return fail(LQ_ERR_UNSUPPORTED, "%s: batch %lld > 16", fn, (long long)b);
    lq_status st = check_wo(fn, 8, x_bf16, b, codes, scales, zeros, n, k, symmetric, group, y);
    if (st != LQ_OK || b == 0 || n == 0) return st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::WoArgs a{static_cast<const uint16_t *>(x_bf16), b, static_cast<const uint8_t *>(codes), scales, zeros,
                 n, k, symmetric, group, y};
    return launched(lq::launch_w8a16_gemv(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status w4a16_gemm(const void *x_bf16, int64_t m, const void *codes, const float *scales, const float *zeros,
                     int64_t n, int64_t k, int symmetric, int64_t group, float *y, void *stream) {
    const char *fn = "w4a16_gemm";
    lq_status st = check_wo(fn, 4, x_bf16, m, codes, scales, zeros, n, k, symmetric, group, y);
    if (st != LQ_OK || m == 0 || n == 0) return st;
    // a 128-row activation tile is addressed with 32-bit buffer offsets
    if (k >= (int64_t(1) << 24)) return fail(LQ_ERR_UNSUPPORTED, "%s: k >= 2^24", fn);
    if ((st = need_device()) != LQ_OK) return st;
    lq::WoArgs a{static_cast<const uint16_t *>(x_bf16), m, static_cast<const uint8_t *>(codes), scales, zeros,
                 n, k, symmetric, group, y};
    return launched(lq::launch_w4a16_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status smooth_scale(const void *x_bf16, int64_t t, const void *w_bf16, int64_t n, int64_t k, float alpha,
                       float *s, void *stream) {
    const char *fn = "smooth_scale";
    if (t <= 0 || n <= 0 || k <= 0)
        return fail(LQ_ERR_INVALID_ARG, "%s: t, n and k must be positive (channel maxima of empty tensors)", fn);
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(LQ_ERR_INVALID_ARG, "%s: alpha must be in [0, 1]", fn);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (t > kMaxDim || n > kMaxDim || k > kMaxDim || n * k > kMaxElems || t * k > kMaxElems)
        return fail(LQ_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!w_bf16 || !aligned(w_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: w null or not 16-byte aligned", fn);
    if (!s || !aligned(s, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: s null or not 16-byte aligned", fn);
    if (any_overlap({{s, k * 4}}, {{x_bf16, t * k * 2}, {w_bf16, n * k * 2}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::SmoothArgs a{static_cast<const uint16_t *>(x_bf16), t, static_cast<const uint16_t *>(w_bf16), n, k, alpha, s};
    return launched(lq::launch_smooth_scale(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status quant_per_token_int8(const void *x_bf16, int64_t t, int64_t k, const float *smooth, int8_t *qx,
                               float *sx, void *stream) {
    const char *fn = "quant_per_token_int8";
    if (t < 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: t must be >= 0 and k > 0", fn);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (t > kMaxDim || k > kMaxDim || t * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    if (t == 0) return LQ_OK;
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (smooth && !aligned(smooth, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: smooth not 16-byte aligned", fn);
    if (!qx || !aligned(qx, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: qx null or not 16-byte aligned", fn);
    if (!sx || !aligned(sx, 4)) return fail(LQ_ERR_INVALID_ARG, "%s: sx null or misaligned", fn);
    if (any_overlap({{qx, t * k}, {sx, t * 4}}, {{x_bf16, t * k * 2}, {smooth, smooth ? k * 4 : 0}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output overlaps an input or another output", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::TokenQuantArgs a{static_cast<const uint16_t *>(x_bf16), t, k, smooth, qx, sx};
    return launched(lq::launch_quant_per_token(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status w8a8_gemm(const int8_t *qx, const float *sx, int64_t m, const int8_t *qw, const float *sw, int64_t n,
                    int64_t k, int32_t *acc, float *y, void *stream) {
    const char *fn = "w8a8_gemm";
    if (m < 0 || n < 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative size or k <= 0", fn);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    // |acc| <= k * 128 * 128 must stay below 2^31: k <= 131071, so at most
    // 130944 (the last multiple of 128 below it)
    if (k > kMaxW8a8K)
        return fail(LQ_ERR_UNSUPPORTED, "%s: k > %lld could overflow the int32 accumulator", fn,
                    (long long)kMaxW8a8K);
    if (m > kMaxDim || n > kMaxDim) return fail(LQ_ERR_UNSUPPORTED, "%s: dimension too large", fn);
    if (m == 0 || n == 0) return LQ_OK;
    if (!qx || !aligned(qx, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: qx null or not 16-byte aligned", fn);
    if (!qw || !aligned(qw, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: qw null or not 16-byte aligned", fn);
    if (!sx || !aligned(sx, 4) || !sw || !aligned(sw, 4))
        return fail(LQ_ERR_INVALID_ARG, "%s: sx/sw null or misaligned", fn);
    if (!y || !aligned(y, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: y null or not 16-byte aligned", fn);
    if (acc && !aligned(acc, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: acc not 16-byte aligned", fn);
    if (any_overlap({{y, m * n * 4}, {acc, acc ? m * n * 4 : 0}},
                    {{qx, m * k}, {qw, n * k}, {sx, m * 4}, {sw, n * 4}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output overlaps an input or another output", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::W8Args a{qx, sx, m, qw, sw, n, k, acc, y};
    return launched(lq::launch_w8a8_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status mxfp4_quantize(const void *w_bf16, int64_t n, int64_t k, void *codes, void *scales, void *stream) {
    const char *fn = "mxfp4_quantize";
    if (n < 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: n must be >= 0 and k > 0", fn);
    if (k % 32 != 0) return fail(LQ_ERR_INVALID_ARG, "%s: k (%lld) is not a multiple of the block of 32", fn,
                                 (long long)k);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (n > kMaxDim || k > kMaxDim || n * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: matrix too large", fn);
    if (n == 0) return LQ_OK;
    if (!w_bf16 || !aligned(w_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: w null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (!scales || !aligned(scales, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: scales null or not 16-byte aligned", fn);
    if (any_overlap({{codes, n * k / 2}, {scales, n * k / 32}}, {{w_bf16, n * k * 2}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output overlaps the input or the other output", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    return launched(lq::launch_mx_quantize(static_cast<const uint16_t *>(w_bf16), n, k, static_cast<uint8_t *>(codes),
                                           static_cast<uint8_t *>(scales), static_cast<hipStream_t>(stream)),
                    fn);
}

lq_status mxfp4_gemv(const void *x_bf16, int64_t b, const void *codes, const void *scales, int64_t n, int64_t k,
                     float *y, void *stream) {
    const char *fn = "mxfp4_gemv";
    if (b < 0 || n < 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative size or k <= 0", fn);
    if (b > 16) return fail(LQ_ERR_UNSUPPORTED, "%s: batch %lld > 16", fn, (long long)b);
    if (k % 32 != 0) return fail(LQ_ERR_INVALID_ARG, "%s: k (%lld) is not a multiple of the block of 32", fn,
                                 (long long)k);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (n > kMaxDim || k > (int64_t(1) << 28)) return fail(LQ_ERR_UNSUPPORTED, "%s: dimension too large", fn);
    if (b == 0 || n == 0) return LQ_OK;
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (!scales || !aligned(scales, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: scales null or not 16-byte aligned", fn);
    if (!y || !aligned(y, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: y null or not 16-byte aligned", fn);
    if (any_overlap({{y, b * n * 4}}, {{x_bf16, b * k * 2}, {codes, n * k / 2}, {scales, n * k / 32}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::MxArgs a{static_cast<const uint16_t *>(x_bf16), b, static_cast<const uint8_t *>(codes),
                 static_cast<const uint8_t *>(scales), n, k, y};
    return launched(lq::launch_mx_gemv(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status mxfp4_gemm(const void *x_bf16, int64_t m, const void *codes, const void *scales, int64_t n, int64_t k,
                     float *y, void *stream) {
    const char *fn = "mxfp4_gemm";
    if (m < 0 || n < 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative size or k <= 0", fn);
    if (k % 32 != 0) return fail(LQ_ERR_INVALID_ARG, "%s: k (%lld) is not a multiple of the block of 32", fn,
                                 (long long)k);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (m > kMaxDim || n > kMaxDim || k >= (int64_t(1) << 24))
        return fail(LQ_ERR_UNSUPPORTED, "%s: dimension too large", fn);
    if (m == 0 || n == 0) return LQ_OK;
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if (!scales || !aligned(scales, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: scales null or not 16-byte aligned", fn);
    if (!y || !aligned(y, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: y null or not 16-byte aligned", fn);
    if (any_overlap({{y, m * n * 4}}, {{x_bf16, m * k * 2}, {codes, n * k / 2}, {scales, n * k / 32}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    lq::MxArgs a{static_cast<const uint16_t *>(x_bf16), m, static_cast<const uint8_t *>(codes),
                 static_cast<const uint8_t *>(scales), n, k, y};
    return launched(lq::launch_mxfp4_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

int64_t gptq_workspace_bytes(int64_t t, int64_t n, int64_t k) {
    if (t < 0 || n < 0 || k <= 0 || t > kMaxDim || n > kMaxDim || k > kMaxDim || k * k > kMaxElems ||
        n * k > kMaxElems || t * k > kMaxElems)
        return -1;
    const int64_t f = t > 0 ? lq::gptq_factor_workspace_bytes(t, k) : 0;
    const int64_t q = n > 0 ? lq::gptq_quantize_workspace_bytes(n, k) : 0;
    return f > q ? f : q;
}

lq_status gptq_hessian_factor(const void *x_bf16, int64_t t, int64_t k, float percdamp, void *workspace,
                              int64_t workspace_bytes, float *u, void *stream) {
    const char *fn = "gptq_hessian_factor";
    if (t <= 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: t and k must be positive", fn);
    if (!(percdamp > 0.0f && percdamp <= 1.0f)) return fail(LQ_ERR_INVALID_ARG, "%s: percdamp must be in (0, 1]", fn);
    if (k % 128 != 0) return fail(LQ_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
    if (t > kMaxDim || k > 65536 || t * k > kMaxElems || t >= (int64_t(1) << 24))
        return fail(LQ_ERR_UNSUPPORTED, "%s: t or k too large", fn);
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!u || !aligned(u, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: u null or not 16-byte aligned", fn);
    const int64_t need = lq::gptq_factor_workspace_bytes(t, k);
    if (!workspace || !aligned(workspace, 256))
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                    (long long)need);
    if (any_overlap({{u, k * k * 4}, {workspace, need}}, {{x_bf16, t * k * 2}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: u or the workspace overlaps x or each other", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    return launched(lq::launch_gptq_factor(static_cast<const uint16_t *>(x_bf16), t, k, percdamp, workspace, u,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

namespace {

// Arguments of the column loop other than its scratch.
lq_status check_gptq_quantize(const char *fn, const void *w_bf16, int64_t n, int64_t k, const float *u, int bits,
                              int symmetric, int64_t group, const void *codes, const float *scales,
                              const float *zeros) {
    if (n < 0) return fail(LQ_ERR_INVALID_ARG, "%s: negative n", fn);
    lq_status st = check_group(fn, k, bits, group);
    if (st != LQ_OK) return st;
    if (n > kMaxDim || k > 65536 || n * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: matrix too large", fn);
    if (n == 0) return LQ_OK;
    if (!w_bf16 || !aligned(w_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: w null or not 16-byte aligned", fn);
    if (!u || !aligned(u, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: u null or not 16-byte aligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    return check_meta(fn, symmetric, scales, zeros);
}

}  // namespace

lq_status gptq_quantize(const void *w_bf16, int64_t n, int64_t k, const float *u, int bits, int symmetric,
                        int64_t group, void *workspace, int64_t workspace_bytes, void *codes, float *scales,
                        float *zeros, void *stream) {
    const char *fn = "gptq_quantize";
    lq_status st = check_gptq_quantize(fn, w_bf16, n, k, u, bits, symmetric, group, codes, scales, zeros);
    if (st != LQ_OK || n == 0) return st;
    const int64_t need = lq::gptq_quantize_workspace_bytes(n, k);
    if (!workspace || !aligned(workspace, 256))
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                    (long long)need);
    const int64_t meta = n * (k / group) * 4;
    const int64_t cbytes = bits == 4 ? n * k / 2 : n * k;
    if (any_overlap({{workspace, need}, {codes, cbytes}, {scales, meta}, {zeros, symmetric ? 0 : meta}},
                    {{w_bf16, n * k * 2}, {u, k * k * 4}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output or the workspace overlaps an input or another output", fn);
    if ((st = need_device()) != LQ_OK) return st;
    lq::GptqArgs a{static_cast<const uint16_t *>(w_bf16), n, k, u, bits, symmetric, group, workspace,
                   static_cast<uint8_t *>(codes), scales, zeros};
    return launched(lq::launch_gptq_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

int64_t gptq_quantize_noalloc_max_bytes(void) { return lq::gptq_static_scratch_bytes(); }

lq_status gptq_quantize_noalloc(const void *w_bf16, int64_t n, int64_t k, const float *u, int bits, int symmetric,
                                int64_t group, void *codes, float *scales, float *zeros, void *stream) {
    const char *fn = "gptq_quantize_noalloc";
    lq_status st = check_gptq_quantize(fn, w_bf16, n, k, u, bits, symmetric, group, codes, scales, zeros);
    if (st != LQ_OK || n == 0) return st;
    const int64_t need = lq::gptq_quantize_workspace_bytes(n, k);
    const int64_t have = lq::gptq_static_scratch_bytes();
    if (need > have)
        return fail(LQ_ERR_UNSUPPORTED,
                    "%s: n = %lld, k = %lld needs %lld bytes of scratch (an fp32 copy of W and the block's "
                    "scaled errors); the static scratch holds %lld. Use gptq_quantize with a workspace",
                    fn, (long long)n, (long long)k, (long long)need, (long long)have);
    const int64_t meta = n * (k / group) * 4;
    const int64_t cbytes = bits == 4 ? n * k / 2 : n * k;
    if (any_overlap({{codes, cbytes}, {scales, meta}, {zeros, symmetric ? 0 : meta}},
                    {{w_bf16, n * k * 2}, {u, k * k * 4}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output overlaps an input or another output", fn);
    if ((st = need_device()) != LQ_OK) return st;
    void *ws = nullptr;
    const hipError_t e = lq::gptq_static_scratch(&ws);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LQ_ERR_HIP, "%s: the static scratch's device address: %s", fn, hipGetErrorString(e));
    }
    lq::GptqArgs a{static_cast<const uint16_t *>(w_bf16), n, k, u, bits, symmetric, group, ws,
                   static_cast<uint8_t *>(codes), scales, zeros};
    return launched(lq::launch_gptq_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

lq_status act_absmean(const void *x_bf16, int64_t t, int64_t k, float *sx, void *stream) {
    const char *fn = "act_absmean";
    if (t <= 0 || k <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: t and k must be positive (a mean of no tokens)", fn);
    if (t > kMaxDim || k > kMaxDim || t * k > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!sx || !aligned(sx, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: sx null or not 16-byte aligned", fn);
    if (any_overlap({{sx, k * 4}}, {{x_bf16, t * k * 2}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: output overlaps the input", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    return launched(lq::launch_act_absmean(static_cast<const uint16_t *>(x_bf16), t, k, sx,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

int64_t awq_workspace_bytes(int64_t t, int64_t n, int64_t k) {
    if (t <= 0 || n <= 0 || k <= 0 || t > kMaxDim || n > kMaxDim || k > kMaxDim || t * n > kMaxElems ||
        t * k > kMaxElems)
        return -1;
    return lq::awq_workspace_bytes(t, n, k);
}

lq_status awq_search(const void *x_bf16, int64_t t, const void *w_bf16, int64_t n, int64_t k, int symmetric,
                     int64_t group, int n_grid, const float *sx, void *workspace, int64_t workspace_bytes,
                     float *s_best, double *losses, int32_t *best, void *codes, float *scales, float *zeros,
                     void *stream) {
    const char *fn = "awq_search";
    if (t <= 0 || n <= 0) return fail(LQ_ERR_INVALID_ARG, "%s: t and n must be positive", fn);
    lq_status st = check_group(fn, k, 4, group);
    if (st != LQ_OK) return st;
    if (n_grid < 1 || n_grid > 1024) return fail(LQ_ERR_INVALID_ARG, "%s: n_grid must be in 1..1024", fn);
    if (t > kMaxDim || n > kMaxDim || t * n > kMaxElems || t * k > kMaxElems || n * k > kMaxElems)
        return fail(LQ_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    // the products address 128-row tiles with 32-bit buffer offsets
    if (k >= (int64_t(1) << 24)) return fail(LQ_ERR_UNSUPPORTED, "%s: k >= 2^24", fn);
    if (!x_bf16 || !aligned(x_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: x null or not 16-byte aligned", fn);
    if (!w_bf16 || !aligned(w_bf16, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: w null or not 16-byte aligned", fn);
    if (!sx || !aligned(sx, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: sx null or not 16-byte aligned", fn);
    const int64_t need = lq::awq_workspace_bytes(t, n, k);
    if (!workspace || !aligned(workspace, 256))
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(LQ_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                    (long long)need);
    if (!s_best || !aligned(s_best, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: s_best null or not 16-byte aligned", fn);
    if (!losses || !aligned(losses, 8)) return fail(LQ_ERR_INVALID_ARG, "%s: losses null or misaligned", fn);
    if (!best || !aligned(best, 4)) return fail(LQ_ERR_INVALID_ARG, "%s: best null or misaligned", fn);
    if (!codes || !aligned(codes, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: codes null or not 16-byte aligned", fn);
    if ((st = check_meta(fn, symmetric, scales, zeros)) != LQ_OK) return st;
    const int64_t meta = n * (k / group) * 4;
    if (any_overlap({{workspace, need}, {s_best, k * 4}, {losses, (int64_t)(n_grid + 1) * 8}, {best, 4},
                     {codes, n * k / 2}, {scales, meta}, {zeros, symmetric ? 0 : meta}},
                    {{x_bf16, t * k * 2}, {w_bf16, n * k * 2}, {sx, k * 4}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: an output or the workspace overlaps an input or another output", fn);
    if ((st = need_device()) != LQ_OK) return st;
    lq::AwqArgs a{static_cast<const uint16_t *>(x_bf16), t, static_cast<const uint16_t *>(w_bf16), n, k,
                  symmetric, group, n_grid, sx, workspace, s_best, losses, best,
                  static_cast<uint8_t *>(codes), scales, zeros};
    return launched(lq::launch_awq_search(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

int64_t lq_read_probe_sink_words(void) { return lq::read_probe_sink_words(); }

lq_status lq_hbm_read_probe(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
    const char *fn = "lq_hbm_read_probe";
    if (bytes < 0 || bytes % 16 != 0) return fail(LQ_ERR_INVALID_ARG, "%s: bytes must be a non-negative multiple of 16", fn);
    if (bytes > kMaxElems) return fail(LQ_ERR_UNSUPPORTED, "%s: buffer too large", fn);
    if (bytes == 0) return LQ_OK;
    if (!p || !aligned(p, 16)) return fail(LQ_ERR_INVALID_ARG, "%s: buffer null or not 16-byte aligned", fn);
    if (!sink || !aligned(sink, 4)) return fail(LQ_ERR_INVALID_ARG, "%s: sink null or misaligned", fn);
    if (any_overlap({{sink, lq::read_probe_sink_words() * 4}}, {{p, bytes}}))
        return fail(LQ_ERR_INVALID_ARG, "%s: the sink overlaps the buffer", fn);
    lq_status st;
    if ((st = need_device()) != LQ_OK) return st;
    return launched(lq::launch_read_probe(p, bytes, sink, static_cast<hipStream_t>(stream)), fn);
}
