// launch.hpp -- argument records passed from the C-ABI layer (api.cpp) to
// the per-kernel launchers. Arguments are validated before they get here.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

struct QuantArgs {
    const uint16_t *w;
    int64_t n, k;
    int bits, symmetric;
    int64_t group;
    const float *col_scale;
    uint8_t *codes;
    float *scales, *zeros;
    // batch of products of the same W under different column scales (the AWQ
    // grid): batch p reads col_scale + p cs_stride and writes codes + p
    // code_stride (bytes), scales and zeros + p meta_stride (floats)
    int batch = 1;
    int64_t cs_stride = 0, code_stride = 0, meta_stride = 0;
};

struct DequantArgs {
    const uint8_t *codes;
    const float *scales, *zeros;
    int64_t n, k;
    int bits, symmetric;
    int64_t group;
    float *out;
};

// Weight-only products (W4A16 and W8A16): bf16 activations, integer codes.
struct WoArgs {
    const uint16_t *x;
    int64_t m;  // batch (GEMV) or tokens (GEMM)
    const uint8_t *codes;
    const float *scales, *zeros;
    int64_t n, k;
    int symmetric;
    int64_t group;
    float *y;
};

struct SmoothArgs {
    const uint16_t *x;
    int64_t t;
    const uint16_t *w;
    int64_t n, k;
    float alpha;
    float *s;
};

struct TokenQuantArgs {
    const uint16_t *x;
    int64_t t, k;
    const float *smooth;
    int8_t *qx;
    float *sx;
};

struct W8Args {
    const int8_t *qx;
    const float *sx;
    int64_t m;
    const int8_t *qw;
    const float *sw;
    int64_t n, k;
    int32_t *acc;
    float *y;
};

// MXFP4 weights (E2M1 codes, E8M0 block scales) with bf16 activations.
struct MxArgs {
    const uint16_t *x;
    int64_t m;
    const uint8_t *codes;
    const uint8_t *scales;
    int64_t n, k;
    float *y;
};

// GPTQ column loop: weights, the inverse-Hessian factor U and the outputs.
struct GptqArgs {
    const uint16_t *w;  // [n][k]
    int64_t n, k;
    const float *u;     // [k][k], upper
    int bits, symmetric;
    int64_t group;
    void *workspace;
    uint8_t *codes;
    float *scales, *zeros;
};

// AWQ scale search (bits 4): inputs, the caller's workspace and outputs.
struct AwqArgs {
    const uint16_t *x;  // calibration activations [t][k]
    int64_t t;
    const uint16_t *w;  // weights [n][k]
    int64_t n, k;
    int symmetric;
    int64_t group;
    int n_grid;
    const float *sx;    // channel mean magnitudes [k]
    void *workspace;
    float *s_best;
    double *losses;     // [n_grid + 1]
    int32_t *best;
    uint8_t *codes;
    float *scales, *zeros;
};

// Decode GEMV at batch 4..16 on large matrices (gemv_shared.hip), for the
// three weight formats. scales: fp32 [n][k / group] for INT4 and INT8,
// E8M0 bytes [n][k / 32] for MXFP4 (group and zeros unused there).
enum class WeightFormat { kInt4, kInt8, kMx };

struct SharedGemvArgs {
    const uint16_t *x;
    int64_t m;
    const uint8_t *codes;
    const void *scales;
    const float *zeros;
    int64_t n, k;
    int symmetric;
    int64_t group;
    float *y;
};

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t st);
hipError_t launch_w4a16_gemv(const WoArgs &a, hipStream_t st);
hipError_t launch_w4a16_gemm(const WoArgs &a, hipStream_t st);
// `points` products of a's shape in one launch, point p's activations,
// codes and scales / zeros at p times the given element strides from a's;
// each workgroup writes sum (yref - y)^2 over its outputs (fp64) to
// loss[p * blocks + block], blocks = w4a16_gemm_blocks(m, n); y is not stored.
int64_t w4a16_gemm_blocks(int64_t m, int64_t n);
hipError_t launch_w4a16_gemm_loss(const WoArgs &a, int points, int64_t x_stride, int64_t code_stride,
                                  int64_t meta_stride, const float *yref, double *loss, hipStream_t st);
hipError_t launch_w8a16_gemv(const WoArgs &a, hipStream_t st);
hipError_t launch_smooth_scale(const SmoothArgs &a, hipStream_t st);
hipError_t launch_quant_per_token(const TokenQuantArgs &a, hipStream_t st);
hipError_t launch_w8a8_gemm(const W8Args &a, hipStream_t st);
hipError_t launch_mx_quantize(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales,
                              hipStream_t st);
hipError_t launch_mx_gemv(const MxArgs &a, hipStream_t st);
hipError_t launch_act_absmean(const uint16_t *x, int64_t t, int64_t k, float *sx, hipStream_t st);
hipError_t launch_awq_search(const AwqArgs &a, hipStream_t st);
int64_t gptq_factor_workspace_bytes(int64_t t, int64_t k);
int64_t gptq_quantize_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_gptq_factor(const uint16_t *x, int64_t t, int64_t k, float percdamp, void *workspace, float *u,
                              hipStream_t st);
hipError_t launch_gptq_quantize(const GptqArgs &a, hipStream_t st);
// The column loop's static device scratch: its size, and its device address
// on the current device (looked up once per device).
int64_t gptq_static_scratch_bytes();
hipError_t gptq_static_scratch(void **ptr);
// Y[m][n] = A[m][k] B[n][k]^T, bf16 inputs (k a multiple of 64), fp32 out.
hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t m, int64_t n, int64_t k, float *y,
                            hipStream_t st);
int64_t awq_workspace_bytes(int64_t t, int64_t n, int64_t k);
// Whether the shared-stage kernel is the faster one for this shape, and its
// launcher (which takes any shape it is given, batch 1..16).
bool shared_gemv_pays(WeightFormat f, int64_t m, int64_t n, int64_t k);
hipError_t launch_shared_gemv(WeightFormat f, const SharedGemvArgs &a, hipStream_t st);

// MXFP4 prefill GEMM (gemm.hip): Y[m][n] = X W^T with MXFP4 weights, any m.
hipError_t launch_mxfp4_gemm(const MxArgs &a, hipStream_t st);

// streaming-read probe (probe.hip)
int64_t read_probe_sink_words();
hipError_t launch_read_probe(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace lq
