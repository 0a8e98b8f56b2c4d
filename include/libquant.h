/*
 * libquant.h -- C ABI of the MI355X (gfx950) library for group-wise
 * round-to-nearest (RTN) quantization, the W4A16 GEMV/GEMM that consumes its
 * packed codes, and the SmoothQuant W8A8 path.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor pointer is a DEVICE pointer on the current HIP
 *           device, allocated and owned by the caller. The library never
 *           allocates, frees or keeps tensor memory, and keeps no state
 *           between calls except a thread-local error string and the one
 *           static device array of gptq_quantize_noalloc (described there).
 * Layout.   Row-major, the last index contiguous. Weights are W[n][k] with
 *           n = output features and k = input features; activations are
 *           X[m][k]. This is the linear layer Y = X W^T with W[out, in] and
 *           per-group parameters along in_features ("LLM quantization deep
 *           dive", rainlib.com, "granularity and matrix dimensions").
 *           bf16 tensors are passed as raw 16-bit patterns (void*).
 *           Packed INT4 codes: [n][k/2] bytes, element 2j in the low nibble
 *           of byte j and element 2j+1 in the high nibble. INT8 codes:
 *           [n][k] bytes. scales / zeros: fp32 [n][k/group].
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL is the null
 *           stream) and the call returns after the launch. Synchronising
 *           is the caller's business. Calls that overlap on one stream are
 *           ordered; calls on different streams that write the same buffer
 *           race.
 * Errors.   Every entry point returns an lq_status. Arguments are checked
 *           before any HIP call. A rejected call enqueues no work and writes
 *           no output. Outputs may not overlap inputs. No exception crosses
 *           the ABI, and the library never prints or exits.
 *           LQ_ERR_INVALID_ARG   null required pointer, negative size, k not a
 *                                multiple of group, zeros given for a
 *                                symmetric call (or missing for an
 *                                asymmetric one), misaligned pointer,
 *                                overlapping input/output ranges.
 *           LQ_ERR_UNSUPPORTED   a well-formed request this build does not
 *                                implement (see each entry point).
 *           LQ_ERR_NO_DEVICE     no HIP device is visible.
 *           LQ_ERR_HIP           a HIP launch failed; lq_last_error() names it.
 *           Empty work (n == 0 or m == 0 / t == 0 / b == 0) is a successful
 *           no-op.
 * Alignment. bf16, code, int8 and output tensors: 16 bytes. fp32 scale,
 *           zero and vector arguments: 4 bytes.
 * Numerics. Inputs must be finite. Codes, scales, zeros, INT8 codes, the
 *           smoothing factors at alpha = 0.5 and the W8A8 int32 accumulators
 *           are bit-exact against the IEEE-fp32 definitions below (correctly
 *           rounded division and square root, round-half-to-even, no FMA
 *           contraction, subnormals kept). Float matmul outputs are fp32
 *           accumulations; they agree with an fp64 evaluation of the same
 *           definition to relative L2 <= 1e-3 and max abs <= 1e-2 max|y|.
 *           One group whose values are all equal and above ~1e29 in magnitude
 *           makes x/s overflow fp32; such groups are outside the contract.
 */
#ifndef LIBQUANT_H
#define LIBQUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LQ_OK = 0,
    LQ_ERR_INVALID_ARG = 1,
    LQ_ERR_UNSUPPORTED = 2,
    LQ_ERR_HIP = 3,
    LQ_ERR_NO_DEVICE = 4
} lq_status;

/* Version of this ABI (incremented on any incompatible change). */
#define LQ_ABI_VERSION 1
int lq_abi_version(void);

/* Static description of a status code (never NULL). */
const char *lq_status_string(lq_status status);

/* Detail of the last failure on the calling thread ("" if none). The string
 * is owned by the library and valid until the next call on this thread. */
const char *lq_last_error(void);

/*
 * quantize_groupwise -- group-wise RTN quantization of W[n][k] along k.
 *
 * Definition ("3.6 Quantization", LLM learning path, section "Symmetric and
 * asymmetric quantization", and its PyTorch code block; same formulas in
 * "Quantization: trading precision for performance", mokono.cn, 2.3/3.3):
 * for each row and each run of `group` consecutive k (x = W, times
 * col_scale[k] in fp32 when col_scale is given):
 *   symmetric : qmax = 2^(bits-1) - 1, s = max(max|x|, 1e-8) / qmax,
 *               q = clamp(round(x / s), -qmax, qmax)
 *   asymmetric: s = max(max x - min x, 1e-8) / (2^bits - 1),
 *               z = round(-min x / s) (as fp32, -0 stored as +0),
 *               q = clamp(round(x / s) + z, 0, 2^bits - 1)
 * round() is round-half-to-even of the correctly rounded fp32 quotient.
 *
 * w_bf16     [n][k] bf16 weights.
 * bits       4 or 8.
 * symmetric  nonzero for symmetric (no zero point).
 * group      group size along k. Supported: any multiple of 128 that
 *            divides k (128 is the usual G; group == k is per-channel, one
 *            scale per output row). Other values: LQ_ERR_UNSUPPORTED.
 * col_scale  nullable fp32 [k]: SmoothQuant's weight-side factor ("3.6
 *            Quantization", section "SmoothQuant": the weight row of input
 *            channel j is multiplied by s_j), applied before the statistics.
 * codes      out. bits 4: [n][k/2] packed nibbles, symmetric codes stored as
 *            q + 8. bits 8: [n][k], int8 q (symmetric) or uint8 q.
 * scales     out fp32 [n][k/group].
 * zeros      out fp32 [n][k/group] for asymmetric; must be NULL for symmetric.
 * k must be a multiple of 128.
 */
lq_status quantize_groupwise(const void *w_bf16, int64_t n, int64_t k, int bits, int symmetric,
                             int64_t group, const float *col_scale, void *codes, float *scales,
                             float *zeros, void *stream);

/*
 * dequantize_groupwise -- x_hat = s (q - z), in fp32 with a single rounding
 * ("3.6 Quantization", asymmetric equation; "Quantization: trading precision
 * for performance" 2.3, dequantization). For symmetric codes z = 0 (INT4
 * codes stored as q + 8 are decoded to q first).
 * codes/scales/zeros as written by quantize_groupwise; out: fp32 [n][k].
 * Same bits / group / k constraints as quantize_groupwise.
 */
lq_status dequantize_groupwise(const void *codes, const float *scales, const float *zeros,
                               int64_t n, int64_t k, int bits, int symmetric, int64_t group,
                               float *out, void *stream);

/*
 * w4a16_gemv -- batch-b decode product with INT4 weights
 * ("LLM quantization deep dive", W4A16: 4-bit weights in memory, 16-bit
 * activations, unpack/dequantize inside the kernel fused with the product,
 * higher-precision accumulation; "3.6 Quantization", weight-only
 * quantization of memory-bound decoding):
 *   y[i][r] = sum_j x[i][j] * (q[r][j] - z[r][j/group]) * s[r][j/group]
 * x_bf16  [b][k] bf16 activations, b in 0..16 (larger: LQ_ERR_UNSUPPORTED;
 *         use w4a16_gemm).
 * codes   [n][k/2] INT4 codes from quantize_groupwise(bits = 4).
 * scales  fp32 [n][k/group]; zeros fp32 [n][k/group] or NULL if symmetric.
 * y       out fp32 [b][n], device memory (coarse-grained: for batch 4..16 on
 *         matrices of about 40M weights and more with few row blocks, the
 *         kernel splits k, zeroes y on `stream` and adds partial sums into
 *         it with float atomics; with more than two such runs the
 *         summation order, and so the last bits of y, can vary from call
 *         to call. Every other case is deterministic).
 * group: multiple of 128 dividing k; k multiple of 128 and at most 2^28.
 */
lq_status w4a16_gemv(const void *x_bf16, int64_t b, const void *codes, const float *scales,
                     const float *zeros, int64_t n, int64_t k, int symmetric, int64_t group,
                     float *y, void *stream);

/*
 * w8a16_gemv -- batch-b decode product with INT8 weights
 * ("LLM quantization deep dive", W/A/KV notation: W8A16 keeps 8-bit weights
 * and 16-bit activations; as for W4A16 the codes are dequantized inside the
 * kernel and multiplied with the activations, higher-precision
 * accumulation):
 *   y[i][r] = sum_j x[i][j] * (q[r][j] - z[r][j/group]) * s[r][j/group]
 * x_bf16  [b][k] bf16 activations, b in 0..16 (larger: LQ_ERR_UNSUPPORTED).
 * codes   [n][k] INT8 codes from quantize_groupwise(bits = 8): int8 q for
 *         symmetric, uint8 q for asymmetric.
 * scales  fp32 [n][k/group]; zeros fp32 [n][k/group] or NULL if symmetric.
 * y       out fp32 [b][n].
 * group: multiple of 128 dividing k; k multiple of 128 and at most 2^28.
 * Errors as w4a16_gemv; x, codes and y must be 16-byte aligned. Batch
 * 4..16 on large matrices splits k as w4a16_gemv does (y zeroed on `stream`,
 * partial sums added with float atomics; more than two runs: the last bits
 * of y can vary from call to call).
 */
lq_status w8a16_gemv(const void *x_bf16, int64_t b, const void *codes, const float *scales,
                     const float *zeros, int64_t n, int64_t k, int symmetric, int64_t group,
                     float *y, void *stream);

/*
 * w4a16_gemm -- prefill-shaped product with INT4 weights, same definition
 * as w4a16_gemv for any m ("LLM quantization deep dive", prefill is
 * compute-bound; "3.6 Quantization", W4A16 does not speed up prefill).
 * Runs on bf16 MFMA with exact integer weight operands and the per-group
 * scale applied in fp32.
 * x_bf16 [m][k]; y out fp32 [m][n]. Other arguments as w4a16_gemv, with
 * k below 2^24 (LQ_ERR_UNSUPPORTED otherwise).
 */
lq_status w4a16_gemm(const void *x_bf16, int64_t m, const void *codes, const float *scales,
                     const float *zeros, int64_t n, int64_t k, int symmetric, int64_t group,
                     float *y, void *stream);

/*
 * smooth_scale -- SmoothQuant migration strength ("3.6 Quantization",
 * section "SmoothQuant"; PTQ concept page, SmoothQuant):
 *   s[j] = max_t |X[t][j]|^alpha / max_r |W[r][j]|^(1 - alpha)
 * with both maxima floored at 1e-8; alpha = 0.5 is evaluated as
 * sqrt(ax) / sqrt(aw) (bit-exact), other alpha with powf (within 1e-6
 * relative).
 * x_bf16 [t][k] calibration activations; w_bf16 [n][k] weights; s out fp32
 * [k]. alpha in [0, 1]. k multiple of 128. The output buffer s is also the
 * kernels' running-maximum workspace while the call runs.
 */
lq_status smooth_scale(const void *x_bf16, int64_t t, const void *w_bf16, int64_t n, int64_t k,
                       float alpha, float *s, void *stream);

/*
 * quant_per_token_int8 -- dynamic per-token symmetric INT8 of the smoothed
 * activations ("3.6 Quantization", SmoothQuant section and code block:
 * X diag(s)^-1, then one scale per token; compendium "Quantization",
 * activation quantization: dynamic per-token):
 *   X'[t][j] = X[t][j] / smooth[j] (fp32, not re-rounded; smooth may be
 *   NULL for no smoothing), sx[t] = max(max_j |X'[t][j]|, 1e-8) / 127,
 *   qx[t][j] = clamp(round(X'[t][j] / sx[t]), -127, 127).
 * x_bf16 [t][k]; qx out int8 [t][k]; sx out fp32 [t]. k multiple of 128.
 */
lq_status quant_per_token_int8(const void *x_bf16, int64_t t, int64_t k, const float *smooth,
                               int8_t *qx, float *sx, void *stream);

/*
 * w8a8_gemm -- INT8 x INT8 GEMM with INT32 accumulation and fp32 rescale
 * (compendium "Quantization", activation quantization: INT8 operands,
 * INT32 accumulation; "3.6 Quantization" code block: per-token activation
 * scale times per-output-channel weight scale):
 *   acc[i][r] = sum_j qx[i][j] * qw[r][j]   (exact in int32: |acc| <= k * 128^2
 *                                           < 2^31 for k <= 130944)
 *   y[i][r]   = (acc[i][r] * sx[i]) * sw[r] in fp32.
 * qx [m][k], qw [n][k] int8; sx fp32 [m]; sw fp32 [n]; acc out int32 [m][n]
 * (nullable); y out fp32 [m][n]. k multiple of 128 and <= 130944 (the largest
 * such k with k * 128^2 < 2^31, so any int8 codes are exact; larger k:
 * LQ_ERR_UNSUPPORTED).
 */
lq_status w8a8_gemm(const int8_t *qx, const float *sx, int64_t m, const int8_t *qw,
                    const float *sw, int64_t n, int64_t k, int32_t *acc, float *y, void *stream);

/*
 * mxfp4_quantize -- MXFP4 block quantization ("3.6 Quantization", number-
 * format table: FP4 E2M1 elements, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, in
 * blocks of 32 sharing an 8-bit power-of-two scale, E8M0, OCP Microscaling;
 * "Granularity": one scale per block of 32; compendium "Microscaling (MX)
 * formats"). Per block of 32 consecutive elements of a row:
 *   e = the smallest integer with max|w| <= 6 * 2^e, clamped to [-127, 127]
 *       (an all-zero block gives -127); scales[.] = e + 127 (E8M0 byte)
 *   c = the E2M1 value nearest to w / 2^e (ties to the even encoding), with
 *       the sign of w; a zero magnitude is stored as +0.
 * w_bf16 [n][k]; codes out [n][k/2] (nibble sign << 3 | exponent << 1 |
 * mantissa, element 2j in the low nibble of byte j); scales out uint8
 * [n][k/32]. All 16-byte aligned. k multiple of 128 (a multiple of 32 that
 * is not: LQ_ERR_UNSUPPORTED; not a multiple of 32: LQ_ERR_INVALID_ARG).
 * Magnitudes above 6 * 2^126 leave the fp32 range when dequantized and are
 * outside the contract.
 */
lq_status mxfp4_quantize(const void *w_bf16, int64_t n, int64_t k, void *codes, void *scales,
                         void *stream);

/*
 * mxfp4_gemv -- batch-b decode product with MXFP4 weights and 16-bit
 * activations (the weight-only product of "LLM quantization deep dive",
 * W4A16, with the MXFP4 weights above):
 *   y[i][r] = sum_j x[i][j] * E2M1(c[r][j]) * 2^(scales[r][j/32] - 127)
 * x_bf16 [b][k], b in 0..16 (larger: LQ_ERR_UNSUPPORTED); codes, scales as
 * mxfp4_quantize writes them; y out fp32 [b][n]. 16-byte aligned; k multiple
 * of 128 and at most 2^28. Batch 4..16 on large matrices splits k as
 * w4a16_gemv does (y zeroed on `stream`, partial sums added with float
 * atomics; more than two runs: the last bits of y can vary from call to
 * call).
 */
lq_status mxfp4_gemv(const void *x_bf16, int64_t b, const void *codes, const void *scales,
                     int64_t n, int64_t k, float *y, void *stream);

/*
 * mxfp4_gemm -- prefill-shaped product with MXFP4 weights and 16-bit
 * activations, same definition as mxfp4_gemv for any m ("3.6 Quantization",
 * number-format table: MXFP4 is FP4 E2M1 elements in blocks of 32 sharing an
 * E8M0 scale, aimed at 4-bit matrix-core GEMMs; "LLM quantization deep
 * dive", prefill is compute-bound):
 *   y[i][r] = sum_j x[i][j] * E2M1(c[r][j]) * 2^(scales[r][j/32] - 127)
 * Runs on bf16 MFMA: each code byte with its block's scale converts to the
 * exact bf16 pair E2M1(c) 2^e, so the products are exact and the sums fp32.
 * x_bf16 [m][k]; codes, scales as mxfp4_quantize writes them; y out fp32
 * [m][n]. 16-byte aligned; k a multiple of 128 and below 2^24 (a multiple of
 * 32 that is not a multiple of 128: LQ_ERR_UNSUPPORTED; not a multiple of
 * 32: LQ_ERR_INVALID_ARG). E2M1(c) 2^e above the bf16 range (code 6 with
 * e = 127) gives inf, as the exact result would.
 */
lq_status mxfp4_gemm(const void *x_bf16, int64_t m, const void *codes, const void *scales, int64_t n, int64_t k,
                     float *y, void *stream);

/*
 * gptq_workspace_bytes -- device workspace gptq_hessian_factor (t tokens, k
 * channels) and gptq_quantize (n rows, k columns) need; the larger of the
 * two (pass t = 0 or n = 0 for one of them). -1 for sizes they would reject.
 */
int64_t gptq_workspace_bytes(int64_t t, int64_t n, int64_t k);

/*
 * gptq_hessian_factor -- the inverse-Hessian factor GPTQ compensates with
 * ("3.6 Quantization", GPTQ section: H = 2 X X^T of the layer's calibration
 * inputs, and the Cholesky form of its inverse):
 *   H = 2 X^T X (X [t][k]: tokens x input channels; bf16 products, fp32 sums)
 *   H_ii += percdamp * mean_i H_ii  (damping: H is singular when t < k)
 *   u = V^-1 with H = V V^T, V upper triangular (the reverse Cholesky factor),
 *       so u is upper triangular with u^T u = H^-1.
 * x_bf16 [t][k] (16-byte aligned); u out fp32 [k][k] (16-byte aligned,
 * zeros below the diagonal). percdamp in (0, 1]; k a multiple of 128 and at
 * most 65536; t below 2^24. workspace: at least gptq_workspace_bytes(t, 0, k)
 * bytes, 256-byte aligned, scratch. If H is not positive definite after
 * damping (e.g. X all zero), u holds NaN. Layers sharing an input (q, k, v)
 * share u.
 */
lq_status gptq_hessian_factor(const void *x_bf16, int64_t t, int64_t k, float percdamp, void *workspace,
                              int64_t workspace_bytes, float *u, void *stream);

/*
 * gptq_quantize -- GPTQ's column loop ("3.6 Quantization", GPTQ section: quantize
 * W one input column at a time in one order for all rows; after column j
 * move the columns not yet quantized to absorb its rounding error, with
 * lazily batched updates; "LLM quantization deep dive", GPTQ steps):
 *   for j = 0 .. k-1, per row:
 *     at a group's first column: s, z from the group's current weights
 *       (the quantize_groupwise formulas);
 *     q_j = the quantize_groupwise code of w_j; d = (w_j - (q_j - z) s) / u_jj;
 *     w_f = fma(-d, u_jf, w_f) for every f > j (in this order).
 * w_bf16 [n][k]; u [k][k] from gptq_hessian_factor; codes/scales/zeros out
 * exactly as quantize_groupwise lays them out (w4a16_gemv and w8a16_gemv
 * consume them). bits 4 or 8; group a multiple of 128 dividing k; k at most
 * 65536. workspace: at least gptq_workspace_bytes(0, n, k) bytes (an fp32
 * copy of W and the block's scaled errors), 256-byte aligned, scratch.
 */
lq_status gptq_quantize(const void *w_bf16, int64_t n, int64_t k, const float *u, int bits, int symmetric,
                        int64_t group, void *workspace, int64_t workspace_bytes, void *codes, float *scales,
                        float *zeros, void *stream);

/*
 * gptq_quantize_noalloc -- gptq_quantize without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or quantization loops, harnesses that forbid
 * hipMalloc. The call itself allocates and frees nothing. Its scratch (the
 * fp32 copy of W and the block's scaled errors, n * k * 4 + n * 512 bytes,
 * each part rounded up to 256) lives in a static device array of
 * gptq_quantize_noalloc_max_bytes() bytes (72 MiB: one 4096 x 4096 linear
 * fits) that every device the library runs on holds until the process ends;
 * larger n * k return LQ_ERR_UNSUPPORTED before any work. Every call on a
 * device uses that device's one array, so calls that overlap on one device
 * (other streams, other threads) race; calls in order on one stream do not.
 * The array keeps the last call's contents; nothing in it needs to start at
 * zero. Arguments, outputs and errors otherwise as gptq_quantize.
 */
int64_t gptq_quantize_noalloc_max_bytes(void);
lq_status gptq_quantize_noalloc(const void *w_bf16, int64_t n, int64_t k, const float *u, int bits, int symmetric,
                                int64_t group, void *codes, float *scales, float *zeros, void *stream);

/*
 * act_absmean -- the per-channel activation magnitude AWQ scales by
 * ("3.6 Quantization", AWQ section: s_X, the average activation magnitude of
 * each input channel over the calibration data; PTQ concept page, AWQ step 1):
 *   sx[j] = (sum_t |X[t][j]|) / t, summed in fp64, rounded once to fp32.
 * x_bf16 [t][k] calibration activations (16-byte aligned); sx out fp32 [k]
 * (16-byte aligned). t, k >= 1.
 */
lq_status act_absmean(const void *x_bf16, int64_t t, int64_t k, float *sx, void *stream);

/*
 * awq_workspace_bytes -- device workspace awq_search needs for these sizes
 * (the fp32 [t][n] reference product; for each of the 11 grid points it
 * evaluates together, the bf16 [t][k] scaled activations, the fp32 [k]
 * scale vector and the packed INT4 codes, scales and zeros of W diag(s);
 * fp64 loss partials), each piece 256-byte aligned; -1 for sizes
 * awq_search would reject as too large or empty.
 */
int64_t awq_workspace_bytes(int64_t t, int64_t n, int64_t k);

/*
 * awq_search -- AWQ activation-aware scaling with INT4 group-wise RTN
 * ("3.6 Quantization", AWQ section: scale the weight input channels that
 * multiply large activations before rounding, y = sum_j (s_j w_j)(x_j / s_j)
 * -> sum_j quant(s_j w_j) x_j / s_j, with s = s_X^alpha and alpha
 * grid-searched over [0, 1] per layer for the smallest output error on the
 * calibration data; 1/s is folded into the preceding operation. PTQ concept
 * page, AWQ steps 2-5: W' = W diag(s), plain RTN of W'):
 *   for i = 0 .. n_grid:  alpha_i = i / n_grid
 *     s_i[j]    = powf(max(sx[j], 1e-8), alpha_i)
 *     losses[i] = || X W^T - bf16(X / s_i) dequant(quant(W diag(s_i)))^T ||_F^2
 *                 (X W^T and the quantized product in fp32, the squares
 *                 summed in fp64)
 *   best = the first i with the smallest loss; s_best = s_best's s_i; codes,
 *   scales, zeros = quantize_groupwise(W, 4, symmetric, group, col_scale =
 *   s_best). A caller folds 1/s_best into the operation that produces X.
 * x_bf16  [t][k] calibration activations; w_bf16 [n][k] weights; sx [k]
 *         from act_absmean (16-byte aligned each).
 * workspace  device memory of at least awq_workspace_bytes(t, n, k) bytes,
 *         256-byte aligned, owned by the caller, scratch only.
 * s_best out fp32 [k] (16-byte aligned); losses out fp64 [n_grid + 1];
 *         best out int32 [1]; codes/scales/zeros out as quantize_groupwise
 *         with bits = 4 (zeros NULL iff symmetric). All device pointers.
 * group: multiple of 128 dividing k; k below 2^24; n_grid in 1..1024.
 * Errors: LQ_ERR_INVALID_ARG for bad sizes, pointers, a short workspace or
 * overlapping buffers; LQ_ERR_UNSUPPORTED for sizes past the limits above.
 */
lq_status awq_search(const void *x_bf16, int64_t t, const void *w_bf16, int64_t n, int64_t k,
                     int symmetric, int64_t group, int n_grid, const float *sx, void *workspace,
                     int64_t workspace_bytes, float *s_best, double *losses, int32_t *best, void *codes,
                     float *scales, float *zeros, void *stream);

/*
 * Measurement helper (not a step of the method).
 *
 * lq_hbm_read_probe -- reads `bytes` bytes at `p` once with a streaming-read
 * kernel and nothing else: the HBM read rate a kernel that only reads
 * reaches on this device, the practical ceiling of the memory-bound kernels
 * above ("3.6 Quantization": batch-1 decode time is the bytes read over the
 * memory bandwidth). p: device buffer, 16-byte aligned; bytes a multiple of
 * 16. sink: device scratch of lq_read_probe_sink_words() uint32 words that
 * the kernel may write (its contents are meaningless). Asynchronous on
 * `stream`; time it with events around the call.
 */
int64_t lq_read_probe_sink_words(void);
lq_status lq_hbm_read_probe(const void *p, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBQUANT_H */
