/*
 * oracle.c -- plain, slow, scalar CPU reference for group-wise RTN
 * quantization, the W4A16 and W8A16 matmuls that consume its packed codes, and the
 * SmoothQuant W8A8 path.
 *
 * THIS FILE IS TEST INFRASTRUCTURE. It is the independent checker for the
 * HIP library: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load it. The product path never calls it, and it shares
 * no code, header, table or helper with the HIP sources.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction, IEEE single-precision division, round-half-to-even
 * rintf under the default rounding mode, subnormals preserved).
 *
 * Sources (the five web pages on LLM post-training quantization):
 *  [LP]  "3.6 Quantization" of the LLM learning path (liuzhe1218.github.io),
 *        sections "Symmetric and asymmetric quantization", "Granularity",
 *        "SmoothQuant", the PyTorch fake-quant code block and the worked
 *        INT4 example.
 *  [MK]  "Quantization: trading precision for performance in inference"
 *        (mokono.cn), section 2.3 "core formulas" and 3.3/3.4 (sym/asym,
 *        granularity).
 *  [RL]  "LLM quantization deep dive" (rainlib.com), "Scale, Zero Point,
 *        Group Size" and "granularity and matrix dimensions" (Y = X W^T,
 *        W[out, in], groups along in_features).
 *  [CP]  PTQ concept page (compassingai.com), "basic quantization formula"
 *        and the SmoothQuant transform.
 *  [CM]  Maths/CS/AI compendium ch.17 "Quantization" (godlockin.github.io),
 *        "the quantization equation" and "activation quantization".
 *
 * Readings taken where the pages leave a step open (each is stated at the
 * function that applies it):
 *  - round() is round-half-to-even (the pages' executable code uses
 *    torch.round / jnp.round);
 *  - asymmetric codes round x/s first, then add z (every page writes
 *    round(x/s) + z);
 *  - range and absmax are floored at 1e-8 before the division ([LP] code);
 *  - z is stored as an fp32 integer value, canonicalised to +0.0;
 *  - symmetric codes lie in [-qmax, qmax], stored offset-binary (q + 8) for
 *    INT4 and as signed int8 for INT8;
 *  - INT4 packing is two codes per byte, low nibble = even input index
 *    (the pages call the packing order implementation-defined);
 *  - scales and zeros are fp32, layout [n][k / group];
 *  - float results of the matmuls are fp64 sums of fp32 dequantized weights
 *    times the bf16 activations.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

#define ORACLE_FLOOR 1e-8f /* the pages' clamp(min=1e-8) on range / absmax */

/* bf16 bits -> fp32: exact (bf16 is the top half of an fp32). */
static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float clampf(float v, float lo, float hi)
{
    if (v < lo) return lo;
    if (v > hi) return hi;
    return v;
}

/* ------------------------------------------------------------------------
 * One group of RTN quantization.
 *
 * [LP] "Symmetric and asymmetric quantization":
 *   symmetric : qmax = 2^(b-1) - 1, s = max|x| / qmax,
 *               q = clamp(round(x / s), -qmax, qmax), x_hat = s q
 *   asymmetric: s = (max x - min x) / (2^b - 1), z = round(-min x / s),
 *               q = clamp(round(x / s) + z, 0, 2^b - 1), x_hat = s (q - z)
 * [LP] code block: range / absmax clamped to at least 1e-8 before dividing.
 * Same formulas: [MK] 2.3 and 3.3, [CP] "basic quantization formula",
 * [CM] "the quantization equation".
 *
 * x: the group's values in fp32 (already multiplied by col_scale when the
 * caller applies SmoothQuant's weight-side scaling). Writes integer codes q
 * (signed for symmetric, [0, 2^b-1] for asymmetric) and the group's s, z.
 * ---------------------------------------------------------------------- */
static void quantize_group(const float *x, int64_t g, int bits, int symmetric,
                           int32_t *q, float *s_out, float *z_out)
{
    if (symmetric) {
        const float qmax = (float)((1 << (bits - 1)) - 1); /* 7 or 127 */
        float a = 0.0f;
        for (int64_t j = 0; j < g; ++j) {
            float v = fabsf(x[j]);
            if (v > a) a = v;
        }
        if (a < ORACLE_FLOOR) a = ORACLE_FLOOR;
        const float s = a / qmax;
        for (int64_t j = 0; j < g; ++j) {
            float r = rintf(x[j] / s);
            q[j] = (int32_t)clampf(r, -qmax, qmax);
        }
        *s_out = s;
        *z_out = 0.0f;
    } else {
        const float qmaxu = (float)((1 << bits) - 1); /* 15 or 255 */
        float mn = x[0], mx = x[0];
        for (int64_t j = 1; j < g; ++j) {
            if (x[j] < mn) mn = x[j];
            if (x[j] > mx) mx = x[j];
        }
        float range = mx - mn;
        if (range < ORACLE_FLOOR) range = ORACLE_FLOOR;
        const float s = range / qmaxu;
        /* round(-min / s); "+ 0.0f" turns a -0.0 into +0.0 */
        const float z = rintf(-mn / s) + 0.0f;
        for (int64_t j = 0; j < g; ++j) {
            float r = rintf(x[j] / s) + z; /* round first, then add z */
            q[j] = (int32_t)clampf(r, 0.0f, qmaxu);
        }
        *s_out = s;
        *z_out = z;
    }
}

/* Storage of one code: INT4 symmetric is offset-binary q + 8 (0..15),
 * INT4 asymmetric is q itself; INT8 symmetric is the int8 bit pattern,
 * INT8 asymmetric is the uint8 value. */
static void store_codes(const int32_t *q, int64_t k, int bits, int symmetric,
                        uint8_t *row_codes)
{
    if (bits == 4) {
        for (int64_t j = 0; j < k; j += 2) {
            uint32_t u0 = (uint32_t)(symmetric ? q[j] + 8 : q[j]);
            uint32_t u1 = (uint32_t)(symmetric ? q[j + 1] + 8 : q[j + 1]);
            row_codes[j / 2] = (uint8_t)((u0 & 0xFu) | ((u1 & 0xFu) << 4));
        }
    } else {
        for (int64_t j = 0; j < k; ++j)
            row_codes[j] = (uint8_t)(symmetric ? (uint8_t)(int8_t)q[j] : (uint8_t)q[j]);
    }
}

static int check_args(int64_t n, int64_t k, int bits, int64_t group)
{
    if (n < 0 || k <= 0 || group <= 0 || k % group != 0) return -1;
    if (bits != 4 && bits != 8) return -1;
    if (bits == 4 && (k % 2 != 0 || group % 2 != 0)) return -1;
    return 0;
}

/* Quantize a row-major fp32 matrix w[n][k] group-wise along k (the input
 * dimension; [RL] "granularity and matrix dimensions", [LP] "Granularity":
 * per-group along the input dimension, G = 128 typical; group == k is
 * per-channel, i.e. one scale per output row).
 * col_scale (nullable, [k]): SmoothQuant's weight-side scaling, the row j of
 * W (in Y = X W, [LP] "SmoothQuant") multiplied by s_j -- in the W[n][k]
 * layout here, column k of w multiplied by col_scale[k] (fp32 product, not
 * re-rounded) before the group statistics.
 * codes: [n][k/2] (bits 4) or [n][k] (bits 8); scales, zeros: [n][k/group];
 * zeros is written only for asymmetric. Returns 0, or -1 on bad arguments. */
int oracle_quantize_f32(const float *w, int64_t n, int64_t k, int bits, int symmetric,
                        int64_t group, const float *col_scale, uint8_t *codes,
                        float *scales, float *zeros)
{
    if (check_args(n, k, bits, group)) return -1;
    const int64_t ng = k / group;
    const int64_t row_bytes = bits == 4 ? k / 2 : k;
    float *x = (float *)malloc(sizeof(float) * (size_t)k);
    int32_t *q = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    if (!x || !q) { free(x); free(q); return -1; }
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < k; ++j) {
            float v = w[r * k + j];
            x[j] = col_scale ? v * col_scale[j] : v;
        }
        for (int64_t gi = 0; gi < ng; ++gi) {
            float s, z;
            quantize_group(x + gi * group, group, bits, symmetric, q + gi * group, &s, &z);
            scales[r * ng + gi] = s;
            if (!symmetric) zeros[r * ng + gi] = z;
        }
        store_codes(q, k, bits, symmetric, codes + r * row_bytes);
    }
    free(x);
    free(q);
    return 0;
}

/* Same, with the weights given as bf16 bit patterns (converted exactly). */
int oracle_quantize_bf16(const uint16_t *w, int64_t n, int64_t k, int bits, int symmetric,
                         int64_t group, const float *col_scale, uint8_t *codes,
                         float *scales, float *zeros)
{
    if (check_args(n, k, bits, group)) return -1;
    float *row = (float *)malloc(sizeof(float) * (size_t)k);
    if (!row) return -1;
    const int64_t ng = k / group;
    const int64_t row_bytes = bits == 4 ? k / 2 : k;
    int rc = 0;
    for (int64_t r = 0; r < n && rc == 0; ++r) {
        for (int64_t j = 0; j < k; ++j) row[j] = bf16_bits_to_f32(w[r * k + j]);
        rc = oracle_quantize_f32(row, 1, k, bits, symmetric, group, col_scale,
                                 codes + r * row_bytes, scales + r * ng,
                                 symmetric ? NULL : zeros + r * ng);
    }
    free(row);
    return rc;
}

/* Integer code q of element j of a packed row: the asymmetric code itself,
 * or the signed symmetric code (stored u - 8 for INT4, the int8 value for
 * INT8), so that the dequantized value is (q - z) * s with z = 0 for
 * symmetric. */
static int32_t load_code(const uint8_t *row_codes, int64_t j, int bits, int symmetric)
{
    if (bits == 4) {
        uint8_t b = row_codes[j / 2];
        int32_t u = (j & 1) ? (b >> 4) : (b & 0xF);
        return symmetric ? u - 8 : u;
    }
    return symmetric ? (int32_t)(int8_t)row_codes[j] : (int32_t)row_codes[j];
}

/* Dequantization, x_hat = s (q - z) ([LP] asymmetric equation; [MK] 2.3;
 * [CM] "the quantization equation"), computed in fp32 as one rounding:
 * fl((float)(q - z) * s). q - z is an exact small integer. out: [n][k]. */
int oracle_dequantize(const uint8_t *codes, const float *scales, const float *zeros,
                      int64_t n, int64_t k, int bits, int symmetric, int64_t group,
                      float *out)
{
    if (check_args(n, k, bits, group)) return -1;
    const int64_t ng = k / group;
    const int64_t row_bytes = bits == 4 ? k / 2 : k;
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t *rc = codes + r * row_bytes;
        for (int64_t j = 0; j < k; ++j) {
            const int64_t gi = j / group;
            const float s = scales[r * ng + gi];
            const float z = symmetric ? 0.0f : zeros[r * ng + gi];
            const float qf = (float)load_code(rc, j, bits, symmetric);
            out[r * k + j] = (qf - z) * s;
        }
    }
    return 0;
}

/* Weight-only matmul with 16-bit activations ([RL] "storage dtype vs compute
 * dtype": W4A16 keeps 4-bit weights and bf16 activations, the kernel
 * dequantizes the weights and multiplies them with the activations,
 * accumulating at higher precision; [RL] "W/A/KV notation": W8A16 is the
 * same with 8-bit weights; [RL] linear layer Y = X W^T with W[out, in]):
 *   y[i][r] = sum_j x[i][j] * x_hat[r][j]
 * with x_hat the fp32 dequantized weights above (oracle_dequantize, row by
 * row), summed in fp64 in index order. x: bf16 bits [m][k]; codes: the
 * packed storage of `bits` (k / 2 bytes a row for INT4, k for INT8);
 * y: fp64 [m][n]. */
int oracle_weight_only_matmul(const uint16_t *x, int64_t m, const uint8_t *codes,
                              const float *scales, const float *zeros, int64_t n, int64_t k,
                              int bits, int symmetric, int64_t group, double *y)
{
    if (check_args(n, k, bits, group) || m < 0) return -1;
    float *wrow = (float *)malloc(sizeof(float) * (size_t)k);
    if (!wrow) return -1;
    const int64_t ng = k / group;
    const int64_t codes_per_row = bits == 4 ? k / 2 : k;
    for (int64_t r = 0; r < n; ++r) {
        oracle_dequantize(codes + r * codes_per_row, scales + r * ng,
                          symmetric ? NULL : zeros + r * ng, 1, k, bits, symmetric, group, wrow);
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)wrow[j];
            y[i * n + r] = acc;
        }
    }
    free(wrow);
    return 0;
}

int oracle_w4a16_matmul(const uint16_t *x, int64_t m, const uint8_t *codes,
                        const float *scales, const float *zeros, int64_t n, int64_t k,
                        int symmetric, int64_t group, double *y)
{
    return oracle_weight_only_matmul(x, m, codes, scales, zeros, n, k, 4, symmetric, group, y);
}

/* SmoothQuant migration strength ([LP] "SmoothQuant"; [CP] SmoothQuant;
 * [MK] SmoothQuant): s_j = max_t |X_tj|^alpha / max |W_j|^(1 - alpha).
 * Input maxima are floored at 1e-8 (the pages' only floor constant; they
 * are silent on an all-zero channel). alpha = 0.5 is taken as two
 * correctly rounded square roots and one division; other alpha use powf. */
void oracle_smooth_scale_from_absmax(const float *ax, const float *aw, int64_t k,
                                     float alpha, float *s)
{
    for (int64_t j = 0; j < k; ++j) {
        float a = ax[j] < ORACLE_FLOOR ? ORACLE_FLOOR : ax[j];
        float b = aw[j] < ORACLE_FLOOR ? ORACLE_FLOOR : aw[j];
        if (alpha == 0.5f)
            s[j] = sqrtf(a) / sqrtf(b);
        else
            s[j] = powf(a, alpha) / powf(b, 1.0f - alpha);
    }
}

/* Channel maxima: ax[j] = max over tokens of |X[t][j]|, aw[j] = max over
 * output rows of |W[r][j]| (input channel j is a column of W[n][k]), then
 * the migration strength above. x: bf16 [t][k]; w: bf16 [n][k]; s: [k]. */
int oracle_smooth_scale(const uint16_t *x, int64_t t, const uint16_t *w, int64_t n,
                        int64_t k, float alpha, float *s)
{
    if (t <= 0 || n <= 0 || k <= 0) return -1;
    float *ax = (float *)calloc((size_t)k, sizeof(float));
    float *aw = (float *)calloc((size_t)k, sizeof(float));
    if (!ax || !aw) { free(ax); free(aw); return -1; }
    for (int64_t i = 0; i < t; ++i)
        for (int64_t j = 0; j < k; ++j) {
            float v = fabsf(bf16_bits_to_f32(x[i * k + j]));
            if (v > ax[j]) ax[j] = v;
        }
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            float v = fabsf(bf16_bits_to_f32(w[r * k + j]));
            if (v > aw[j]) aw[j] = v;
        }
    oracle_smooth_scale_from_absmax(ax, aw, k, alpha, s);
    free(ax);
    free(aw);
    return 0;
}

/* Dynamic per-token symmetric INT8 of the smoothed activations
 * ([LP] "SmoothQuant": X diag(s)^-1, i.e. input channel j divided by s_j;
 * [LP] code: quant_sym(X, 8, dim=1), one scale per token; [CM] "activation
 * quantization": dynamic, per-token). X' = X / s in fp32 (not re-rounded),
 * sx = max(max_j |X'_j|, 1e-8) / 127, qx = clamp(round(X' / sx), -127, 127).
 * x: fp32 [t][k]; smooth nullable [k]; qx: [t][k]; sx: [t]. */
int oracle_quant_per_token_int8_f32(const float *x, int64_t t, int64_t k,
                                    const float *smooth, int8_t *qx, float *sx)
{
    if (t < 0 || k <= 0) return -1;
    float *row = (float *)malloc(sizeof(float) * (size_t)k);
    if (!row) return -1;
    for (int64_t i = 0; i < t; ++i) {
        float a = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float v = x[i * k + j];
            row[j] = smooth ? v / smooth[j] : v;
            float av = fabsf(row[j]);
            if (av > a) a = av;
        }
        if (a < ORACLE_FLOOR) a = ORACLE_FLOOR;
        const float s = a / 127.0f;
        for (int64_t j = 0; j < k; ++j)
            qx[i * k + j] = (int8_t)(int32_t)clampf(rintf(row[j] / s), -127.0f, 127.0f);
        sx[i] = s;
    }
    free(row);
    return 0;
}

/* Same with bf16 activations (converted exactly). */
int oracle_quant_per_token_int8(const uint16_t *x, int64_t t, int64_t k,
                                const float *smooth, int8_t *qx, float *sx)
{
    if (t < 0 || k <= 0) return -1;
    float *row = (float *)malloc(sizeof(float) * (size_t)k);
    if (!row) return -1;
    int rc = 0;
    for (int64_t i = 0; i < t && rc == 0; ++i) {
        for (int64_t j = 0; j < k; ++j) row[j] = bf16_bits_to_f32(x[i * k + j]);
        rc = oracle_quant_per_token_int8_f32(row, 1, k, smooth, qx + i * k, sx + i);
    }
    free(row);
    return rc;
}

/* W8A8 INT8 GEMM with INT32 accumulation and fp32 rescale ([CM] "activation
 * quantization": INT8 weights and activations, INT32 accumulation; [LP]
 * code: per-token activation scale times per-output-channel weight scale).
 * acc[i][r] = sum_j qx[i][j] * qw[r][j] (exact int32 for |acc| < 2^31;
 * the sum is formed in int64 and narrowed), y[i][r] = acc * sx[i] * sw[r]
 * in fp64. acc nullable. */
int oracle_w8a8_gemm(const int8_t *qx, const float *sx, int64_t m, const int8_t *qw,
                     const float *sw, int64_t n, int64_t k, int32_t *acc, double *y)
{
    if (m < 0 || n < 0 || k <= 0) return -1;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t r = 0; r < n; ++r) {
            int64_t a = 0;
            for (int64_t j = 0; j < k; ++j)
                a += (int64_t)qx[i * k + j] * (int64_t)qw[r * k + j];
            if (acc) acc[i * n + r] = (int32_t)a;
            y[i * n + r] = (double)a * (double)sx[i] * (double)sw[r];
        }
    return 0;
}

/* Effective bits per weight ([MK] 3.4: 4 + 32/128 = 4.25 for a 16-bit scale
 * and a 16-bit zero per 128 weights; [LP] "Granularity": 16/128 = 0.125 extra
 * bits for a 16-bit scale; [LP] self-test: 4 + (16 + 4)/64 = 4.3125):
 * metadata bits shared by a group are spread over its members. */
double oracle_effective_bits(int bits, int scale_bits, int zero_bits, int64_t group)
{
    return (double)bits + (double)(scale_bits + zero_bits) / (double)group;
}

/* Bytes of the packed layout this library stores for an n x k matrix:
 * codes + fp32 scales + fp32 zeros (asymmetric only). */
int64_t oracle_packed_bytes(int64_t n, int64_t k, int bits, int symmetric, int64_t group)
{
    const int64_t codes = bits == 4 ? n * k / 2 : n * k;
    const int64_t meta = n * (k / group) * 4 * (symmetric ? 1 : 2);
    return codes + meta;
}

/* ------------------------------------------------------------------------
 * AWQ activation-aware scaling ([LP] "AWQ: protecting salient channels by
 * scaling"; [CP] AWQ, steps 1-5; [RL] section 5, activation-aware).
 *
 * A weight input channel j that multiplies large activations is protected
 * by scaling it up before RTN and the activation down by the same factor:
 *   y = sum_j (s_j w_j)(x_j / s_j)  ->  sum_j quant(s_j w_j) x_j / s_j.
 * [LP]: s = s_X^alpha with s_X the mean activation magnitude of each input
 * channel over the calibration data, alpha chosen per layer by a grid
 * search over [0, 1] that minimises the layer's output error on that data;
 * 1/s is folded into the preceding operation.
 * Readings (the pages leave these open):
 *  - the grid is alpha_i = i / n_grid, i = 0 .. n_grid (both ends of [0, 1]);
 *  - s_X is floored at 1e-8 (the pages' only floor constant) before the
 *    power, so a silent channel gives a finite scale;
 *  - the scaled weights are quantized group-wise exactly as quantize_groupwise
 *    does with col_scale = s (fp32 product, not re-rounded);
 *  - the activations reach the quantized product as bf16(x / s): the
 *    preceding operation, with 1/s folded in, emits bf16;
 *  - output error = squared Frobenius norm of X W^T - X' W_hat'^T over the
 *    calibration tokens, in fp64 (X W^T from the bf16 inputs, exact products);
 *  - ties between grid points keep the smallest alpha.
 * ---------------------------------------------------------------------- */

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* s_X[j] = (sum_t |X[t][j]|) / t: the sum in fp64 in token order, divided in
 * fp64 and rounded once to fp32. x: bf16 bits [t][k]. */
int oracle_act_absmean(const uint16_t *x, int64_t t, int64_t k, float *sx)
{
    if (t <= 0 || k <= 0) return -1;
    for (int64_t j = 0; j < k; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < t; ++i) acc += fabs((double)bf16_bits_to_f32(x[i * k + j]));
        sx[j] = (float)(acc / (double)t);
    }
    return 0;
}

/* The candidate scale of grid point i: powf(max(s_X, 1e-8), i / n_grid). */
void oracle_awq_scale(const float *sx, int64_t k, int i, int n_grid, float *s)
{
    const float alpha = (float)i / (float)n_grid;
    for (int64_t j = 0; j < k; ++j) {
        const float v = sx[j] < ORACLE_FLOOR ? ORACLE_FLOOR : sx[j];
        s[j] = powf(v, alpha);
    }
}

/* Output error of one scale vector s [k] against y_ref = X W^T [t][n]. */
static int awq_loss_given_ref(const uint16_t *x, int64_t t, const uint16_t *w, int64_t n, int64_t k,
                              int bits, int symmetric, int64_t group, const float *s,
                              const double *y_ref, double *loss)
{
    const int64_t ng = k / group;
    const int64_t code_bytes = bits == 4 ? n * k / 2 : n * k;
    uint8_t *codes = (uint8_t *)malloc((size_t)code_bytes);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(n * ng));
    float *zr = (float *)malloc(sizeof(float) * (size_t)(n * ng));
    float *w_hat = (float *)malloc(sizeof(float) * (size_t)(n * k));
    float *xs = (float *)malloc(sizeof(float) * (size_t)(t * k));
    int rc = -1;
    if (!codes || !sc || !zr || !w_hat || !xs) goto out;
    /* W' = quant(W diag(s)), dequantized */
    if (oracle_quantize_bf16(w, n, k, bits, symmetric, group, s, codes, sc, zr)) goto out;
    if (oracle_dequantize(codes, sc, symmetric ? NULL : zr, n, k, bits, symmetric, group, w_hat)) goto out;
    /* X' = bf16(X / s) */
    for (int64_t i = 0; i < t; ++i)
        for (int64_t j = 0; j < k; ++j)
            xs[i * k + j] = bf16_bits_to_f32(f32_to_bf16_rne(bf16_bits_to_f32(x[i * k + j]) / s[j]));
    double total = 0.0;
    for (int64_t i = 0; i < t; ++i)
        for (int64_t r = 0; r < n; ++r) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j) acc += (double)xs[i * k + j] * (double)w_hat[r * k + j];
            const double d = y_ref[i * n + r] - acc;
            total += d * d;
        }
    *loss = total;
    rc = 0;
out:
    free(codes); free(sc); free(zr); free(w_hat); free(xs);
    return rc;
}

static double *awq_reference_output(const uint16_t *x, int64_t t, const uint16_t *w, int64_t n, int64_t k)
{
    double *y = (double *)malloc(sizeof(double) * (size_t)(t * n));
    if (!y) return NULL;
    for (int64_t i = 0; i < t; ++i)
        for (int64_t r = 0; r < n; ++r) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)bf16_bits_to_f32(w[r * k + j]);
            y[i * n + r] = acc;
        }
    return y;
}

/* Output error of a given scale vector s [k] (one grid point, or any s). */
int oracle_awq_loss(const uint16_t *x, int64_t t, const uint16_t *w, int64_t n, int64_t k, int bits,
                    int symmetric, int64_t group, const float *s, double *loss)
{
    if (check_args(n, k, bits, group) || t <= 0) return -1;
    double *y_ref = awq_reference_output(x, t, w, n, k);
    if (!y_ref) return -1;
    const int rc = awq_loss_given_ref(x, t, w, n, k, bits, symmetric, group, s, y_ref, loss);
    free(y_ref);
    return rc;
}

/* The search: s_X, the loss of every grid point (losses [n_grid + 1]), the
 * first grid point with the smallest loss (best) and its scale (s_best [k]). */
int oracle_awq_search(const uint16_t *x, int64_t t, const uint16_t *w, int64_t n, int64_t k, int bits,
                      int symmetric, int64_t group, int n_grid, float *sx, double *losses, int *best,
                      float *s_best)
{
    if (check_args(n, k, bits, group) || t <= 0 || n <= 0 || n_grid < 1) return -1;
    if (oracle_act_absmean(x, t, k, sx)) return -1;
    double *y_ref = awq_reference_output(x, t, w, n, k);
    float *s = (float *)malloc(sizeof(float) * (size_t)k);
    int rc = -1;
    if (!y_ref || !s) goto out;
    int arg = 0;
    for (int i = 0; i <= n_grid; ++i) {
        oracle_awq_scale(sx, k, i, n_grid, s);
        if (awq_loss_given_ref(x, t, w, n, k, bits, symmetric, group, s, y_ref, &losses[i])) goto out;
        if (losses[i] < losses[arg]) arg = i;
    }
    *best = arg;
    oracle_awq_scale(sx, k, arg, n_grid, s_best);
    rc = 0;
out:
    free(y_ref); free(s);
    return rc;
}

/* ------------------------------------------------------------------------
 * MXFP4 ([LP] number-format table: FP4 E2M1 elements, magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6, in blocks of 32 sharing one 8-bit power-of-two scale
 * (E8M0), the OCP Microscaling format, about 4.25 bits per element; [LP]
 * "Granularity": one scale per block of 32; [CM] "Microscaling (MX)
 * formats": a block shares an exponent, each element keeps its own bits).
 * Readings (the pages leave these open):
 *  - a block is 32 consecutive elements of a row along k;
 *  - the shared scale is the smallest power of two 2^e with
 *    amax <= 6 * 2^e (the absmax rule s = amax / qmax restricted to powers
 *    of two, so no element clips), e clamped to [-127, 127] (E8M0 = e + 127;
 *    an all-zero block takes e = -127);
 *  - each element is x / 2^e rounded to the nearest E2M1 magnitude, ties to
 *    the even encoding (mantissa bit 0), with the sign of x; a zero
 *    magnitude is stored as +0;
 *  - codes pack two per byte, element 2j in the low nibble (as INT4);
 *    the E2M1 nibble is sign << 3 | exponent << 1 | mantissa.
 * ---------------------------------------------------------------------- */
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* The shared exponent of a block with largest magnitude amax. */
int oracle_mx_exponent(float amax)
{
    if (!(amax > 0.0f)) return -127;
    int p;
    const float m = frexpf(amax, &p);      /* amax = m 2^p, m in [0.5, 1) */
    int e = p - 3 + (m > 0.75f ? 1 : 0);    /* smallest e with amax <= 1.5 * 2^(e + 2) */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Nearest E2M1 magnitude index of a magnitude v in [0, 6], ties to even. */
static int e2m1_round(float v)
{
    int best = 0;
    for (int i = 1; i < 8; ++i) {
        const float d = fabsf(v - kE2M1[i]), db = fabsf(v - kE2M1[best]);
        if (d < db || (d == db && (i & 1) == 0)) best = i;
    }
    return best;
}

/* w: bf16 bits [n][k] (k a multiple of 32); codes [n][k/2]; scales [n][k/32] (E8M0). */
int oracle_mx_quantize(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales)
{
    if (n < 0 || k <= 0 || k % 32 != 0) return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 32; ++b) {
            const uint16_t *x = w + r * k + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                const float a = fabsf(bf16_bits_to_f32(x[j]));
                if (a > amax) amax = a;
            }
            const int e = oracle_mx_exponent(amax);
            scales[r * (k / 32) + b] = (uint8_t)(e + 127);
            uint8_t nib[32];
            for (int j = 0; j < 32; ++j) {
                const float v = bf16_bits_to_f32(x[j]);
                const int mag = e2m1_round(fabsf(ldexpf(v, -e)));
                nib[j] = (uint8_t)(mag == 0 ? 0 : ((v < 0.0f ? 8 : 0) | mag));
            }
            for (int j = 0; j < 32; j += 2)
                codes[r * (k / 2) + b * 16 + j / 2] = (uint8_t)(nib[j] | (nib[j + 1] << 4));
        }
    return 0;
}

/* x_hat = (+-E2M1) * 2^e, exact in fp32. out: [n][k]. */
int oracle_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, float *out)
{
    if (n < 0 || k <= 0 || k % 32 != 0) return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            const uint8_t byte = codes[r * (k / 2) + j / 2];
            const int c = (j & 1) ? byte >> 4 : byte & 0xF;
            const int e = (int)scales[r * (k / 32) + j / 32] - 127;
            const float mag = ldexpf(kE2M1[c & 7], e);
            out[r * k + j] = (c & 8) ? -mag : mag;
        }
    return 0;
}

/* MXFP4 weights with 16-bit activations: y[i][r] = sum_j x[i][j] x_hat[r][j]
 * in fp64 (the weight-only product of the W4A16 rows with MXFP4 weights). */
int oracle_mx_matmul(const uint16_t *x, int64_t m, const uint8_t *codes, const uint8_t *scales, int64_t n,
                     int64_t k, double *y)
{
    if (m < 0 || n < 0 || k <= 0 || k % 32 != 0) return -1;
    float *mrow = (float *)malloc(sizeof(float) * (size_t)k);
    if (!mrow) return -1;
    for (int64_t r = 0; r < n; ++r) {
        oracle_mx_dequantize(codes + r * (k / 2), scales + r * (k / 32), 1, k, mrow);
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j) acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)mrow[j];
            y[i * n + r] = acc;
        }
    }
    free(mrow);
    return 0;
}

/* ------------------------------------------------------------------------
 * GPTQ ([LP] "GPTQ: compensating the error just made"; [RL] GPTQ steps;
 * [CP] GPTQ). Per layer, on calibration data X, minimise ||W X - W_hat X||^2
 * by quantizing W column by column and, after column j (error
 * e_j = w_j - quant(w_j)), moving the not yet quantized columns F:
 *   W[:, F] -= e_j / [H^-1]_jj * [H^-1]_{j, F},   H = 2 X X^T,
 * with the shared column order, lazy batched updates and the Cholesky form
 * the pages name. In the Cholesky form, with U the upper Cholesky factor of
 * H^-1 (U^T U = H^-1), the update of column j is
 *   d = (w_j - w_hat_j) / U_jj,   w_f -= d * U_jf for every f > j.
 * Readings (the pages leave these open):
 *  - X is [t][k] (tokens x input channels), so H = 2 X^T X is [k][k];
 *  - H is damped before inversion: H_ii += 0.01 * mean_i(H_ii) (H is singular
 *    when t < k; the pages give no damping value);
 *  - U is computed from the reverse Cholesky factor V of H (H = V V^T, V upper)
 *    as U = V^-1, in fp64, then rounded to fp32;
 *  - the weights are updated in fp32, each column's update applied to every
 *    later column as one fused multiply-add, in column order (the lazy
 *    batches regroup these updates but keep their order);
 *  - groups follow quantize_groupwise: a group's scale and zero are taken
 *    from the current (already compensated) weights of the group when its
 *    first column is reached; codes round as RTN does.
 * ---------------------------------------------------------------------- */

/* H = 2 X^T X in fp64 (products of bf16 values are exact). x: [t][k].
 * The columns of X are copied out first (xt[i][r] = X[r][i]) so that each
 * sum runs over contiguous memory; the sums are the same, in the same order. */
int oracle_gptq_hessian(const uint16_t *x, int64_t t, int64_t k, double *h)
{
    if (t <= 0 || k <= 0) return -1;
    double *xt = (double *)malloc(sizeof(double) * (size_t)(t * k));
    if (!xt) return -1;
    for (int64_t r = 0; r < t; ++r)
        for (int64_t i = 0; i < k; ++i) xt[i * t + r] = (double)bf16_bits_to_f32(x[r * k + i]);
    for (int64_t i = 0; i < k; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            const double *a = xt + i * t, *b = xt + j * t;
            double acc = 0.0;
            for (int64_t r = 0; r < t; ++r) acc += a[r] * b[r];
            h[i * k + j] = h[j * k + i] = 2.0 * acc;
        }
    free(xt);
    return 0;
}

/* Damping (percdamp of the mean diagonal added to the diagonal), then U:
 * V upper with H = V V^T (reverse Cholesky, last index first), U = V^-1.
 * h is overwritten by the damped H. u: fp32 [k][k], lower triangle zero.
 * Returns -1 if H is not positive definite after damping. */
int oracle_gptq_inverse_factor(double *h, int64_t k, double percdamp, float *u)
{
    if (k <= 0) return -1;
    double mean = 0.0;
    for (int64_t i = 0; i < k; ++i) mean += h[i * k + i];
    mean /= (double)k;
    for (int64_t i = 0; i < k; ++i) h[i * k + i] += percdamp * mean;
    double *v = (double *)calloc((size_t)(k * k), sizeof(double));
    double *w = (double *)calloc((size_t)(k * k), sizeof(double));
    int rc = -1;
    if (!v || !w) goto out;
    /* reverse Cholesky: for j = k-1 .. 0, using the columns right of j */
    for (int64_t j = k - 1; j >= 0; --j) {
        double d = h[j * k + j];
        for (int64_t c = j + 1; c < k; ++c) d -= v[j * k + c] * v[j * k + c];
        if (!(d > 0.0)) goto out;
        const double vjj = sqrt(d);
        v[j * k + j] = vjj;
        for (int64_t i = 0; i < j; ++i) {
            double s = h[i * k + j];
            for (int64_t c = j + 1; c < k; ++c) s -= v[i * k + c] * v[j * k + c];
            v[i * k + j] = s / vjj;
        }
    }
    /* W = V^-1 (upper): back substitution, column by column. Column c of W
     * is kept as row c of wt (wt[c][m] = W[m][c]) so the sums run over
     * contiguous memory. */
    double *wt = w;
    for (int64_t c = 0; c < k; ++c) {
        wt[c * k + c] = 1.0 / v[c * k + c];
        for (int64_t i = c - 1; i >= 0; --i) {
            double s = 0.0;
            for (int64_t m = i + 1; m <= c; ++m) s += v[i * k + m] * wt[c * k + m];
            wt[c * k + i] = -s / v[i * k + i];
        }
    }
    for (int64_t i = 0; i < k; ++i)
        for (int64_t c = 0; c < k; ++c) u[i * k + c] = (float)wt[c * k + i];
    rc = 0;
out:
    free(v);
    free(w);
    return rc;
}

/* The column loop, given U (fp32 [k][k], upper). w: bf16 [n][k]; outputs as
 * oracle_quantize_f32. Rows are independent. */
int oracle_gptq_quantize(const uint16_t *w, int64_t n, int64_t k, const float *u, int bits, int symmetric,
                         int64_t group, uint8_t *codes, float *scales, float *zeros)
{
    if (check_args(n, k, bits, group)) return -1;
    const int64_t ng = k / group;
    const int64_t row_bytes = bits == 4 ? k / 2 : k;
    float *row = (float *)malloc(sizeof(float) * (size_t)k);
    int32_t *q = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    int32_t *qg = (int32_t *)malloc(sizeof(int32_t) * (size_t)group);
    if (!row || !q || !qg) { free(row); free(q); free(qg); return -1; }
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < k; ++j) row[j] = bf16_bits_to_f32(w[r * k + j]);
        float s = 1.0f, z = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            if (j % group == 0) {
                /* this group's scale and zero from its current weights */
                quantize_group(row + j, group, bits, symmetric, qg, &s, &z);
                scales[r * ng + j / group] = s;
                if (!symmetric) zeros[r * ng + j / group] = z;
            }
            /* the code of column j: the RTN formulas with the group's s, z */
            float qf;
            if (symmetric) {
                const float top = (float)((1 << (bits - 1)) - 1); /* 7 or 127 */
                qf = clampf(rintf(row[j] / s), -top, top);
            } else {
                const float top = (float)((1 << bits) - 1);       /* 15 or 255 */
                qf = clampf(rintf(row[j] / s) + z, 0.0f, top);
            }
            q[j] = (int32_t)qf;
            const float w_hat = (qf - z) * s;
            const float d = (row[j] - w_hat) / u[j * k + j];
            for (int64_t f = j + 1; f < k; ++f) row[f] = fmaf(-d, u[j * k + f], row[f]);
        }
        store_codes(q, k, bits, symmetric, codes + r * row_bytes);
    }
    free(row); free(q); free(qg);
    return 0;
}
