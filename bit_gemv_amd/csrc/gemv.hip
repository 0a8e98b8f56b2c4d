// gemv.hip -- W4A16 decode GEMV on gfx950 VALU (v_dot2_f32_bf16).
//
// Definition ("LLM quantization deep dive", rainlib.com, W4A16: INT4 weights
// in memory, unpacked and dequantized inside the kernel and multiplied with
// 16-bit activations, higher-precision accumulation):
//   y[b][r] = sum_j x[b][j] * (q[r][j] - z[r][j/G]) * s[r][j/G].
// At batch 1-16 the product is bound by the bytes of codes and scales
// streamed from HBM ("3.6 Quantization": batch-1 decode time is bytes read
// over bandwidth), so the kernel is built around one coalesced 16-byte code
// load per lane and a small VALU budget per weight:
//
//  * A nibble c ORed into the mantissa of the bf16 0x4300 (= 128) gives the
//    bf16 value 128 + c exactly, so one v_and_or_b32 turns two nibbles of a
//    code word into a packed bf16 pair, and one v_dot2_f32_bf16 multiplies
//    that pair with a pair of activations (exact products, fp32 sums).
//  * The offset and the zero point are folded into a per-segment correction:
//    sum x (q - z) s = s * (sum x (128 + q) - (128 + z) * sum x), where the
//    activation sum comes from the same dot2 unit with a (1, 1) pair.
//  * Nibbles 0..3 of a code word pair with nibbles 4..7, so the activations
//    are re-paired (x0, x4), (x1, x5), ... once per lane and reused over
//    every row the lane visits.
//
// Work split: a lane owns 32 consecutive input elements (16 bytes of codes)
// of a 2048-wide chunk of k; the 4 waves of a block split the chunks of k
// (ks_count ways) and/or the block's rows; partial sums are reduced across
// the wave with butterflies and across waves through LDS. No atomics, so
// results are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kNib = 0x000F000Fu;
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)
constexpr int kChunk = 2048;              // k per wave-wide 16-byte load

// 8 consecutive bf16 activations [x0 x1][x2 x3][x4 x5][x6 x7] -> pairs in
// the order the nibble extraction produces: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
LQ_DEVICE void pair_x(const u32x4 v, uint32_t *p) {
    p[0] = (v.x & 0xFFFFu) | (v.z << 16);
    p[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p[2] = (v.y & 0xFFFFu) | (v.w << 16);
    p[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
}

// One code word (element i of 8 at bits 4i..4i+3) against its 4 x pairs.
LQ_DEVICE float dot8(uint32_t w, const uint32_t *xp, float acc) {
    acc = dot2_bf16((w & kNib) | kMagic, xp[0], acc);
    acc = dot2_bf16(((w >> 4) & kNib) | kMagic, xp[1], acc);
    acc = dot2_bf16(((w >> 8) & kNib) | kMagic, xp[2], acc);
    acc = dot2_bf16(((w >> 12) & kNib) | kMagic, xp[3], acc);
    return acc;
}

// B: batch; RW: rows per wave-set; U: rows in flight per step.
template <int B, int RW, int U, bool SYM>
__global__ __launch_bounds__(256) void gemv_w4_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ codes,
                                                       const float *__restrict__ scales,
                                                       const float *__restrict__ zeros, int n, int k,
                                                       int group, int ks_count,
                                                       float *__restrict__ y) {
    static_assert(RW % U == 0, "rows per wave-set must be a multiple of U");
    __shared__ float red[4][RW * B];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ks = wave % ks_count;
    const int rs = wave / ks_count;
    const int rsets = 4 / ks_count;
    const int row0 = blockIdx.x * (rsets * RW) + rs * RW;
    const int ng = k / group;
    const int nchunks = (k + kChunk - 1) / kChunk;
    const int64_t row_bytes = k / 2;

    float res[RW][B];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) res[r][b] = 0.0f;

    for (int c = ks; c < nchunks; c += ks_count) {
        const int k0 = c * kChunk + lane * 32;
        const bool kv = k0 < k;
        uint32_t xp[B][16];
        float xs[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            xs[b] = 0.0f;
            if (kv) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (int64_t)b * k + k0);
#pragma unroll
                for (int j = 0; j < 4; ++j) pair_x(src[j], &xp[b][4 * j]);
#pragma unroll
                for (int j = 0; j < 16; ++j) xs[b] = dot2_bf16(xp[b][j], kOnes, xs[b]);
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) xp[b][j] = 0u;
            }
        }
        const int gk = k0 / group;
#pragma unroll
        for (int rb = 0; rb < RW; rb += U) {
            u32x4 cw[U];
            float sc[U], zc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = row0 + rb + u;
                if (kv && row < n) {
                    cw[u] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(codes + (int64_t)row * row_bytes + k0 / 2));
                    sc[u] = scales[(int64_t)row * ng + gk];
                    zc[u] = SYM ? 136.0f : 128.0f + zeros[(int64_t)row * ng + gk];
                } else {
                    cw[u] = u32x4{0u, 0u, 0u, 0u};
                    sc[u] = 0.0f;
                    zc[u] = 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float d = 0.0f;
                    d = dot8(cw[u].x, &xp[b][0], d);
                    d = dot8(cw[u].y, &xp[b][4], d);
                    d = dot8(cw[u].z, &xp[b][8], d);
                    d = dot8(cw[u].w, &xp[b][12], d);
                    const float part = sc[u] * __builtin_fmaf(-zc[u], xs[b], d);
                    res[rb + u][b] += team_sum<64>(part);
                }
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) red[wave][r * B + b] = res[r][b];
    }
    __syncthreads();
    if (ks == 0 && lane < RW * B) {
        float v = 0.0f;
        for (int w = 0; w < ks_count; ++w) v += red[rs * ks_count + w][lane];
        const int r = lane / B, b = lane % B;
        const int row = row0 + r;
        if (row < n) y[(int64_t)b * n + row] = v;
    }
}

template <int B, bool SYM>
static hipError_t launch_gemv_b(const W4Args &a, hipStream_t st) {
    constexpr int RW = B == 1 ? 8 : (B <= 4 ? 4 : (B <= 8 ? 2 : 1));
    constexpr int U = RW < 4 ? RW : 4;
    const int nchunks = (int)((a.k + kChunk - 1) / kChunk);
    const int ks_count = nchunks >= 4 ? 4 : (nchunks >= 2 ? 2 : 1);
    const int rows_per_block = (4 / ks_count) * RW;
    const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_w4_kernel<B, RW, U, SYM>), dim3((uint32_t)blocks), dim3(256), 0, st, a.x,
                       a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, ks_count, a.y);
    return hipGetLastError();
}

template <bool SYM>
static hipError_t launch_gemv_s(const W4Args &a, hipStream_t st) {
    switch (a.m) {
#define LQ_B(BB) \
    case BB: return launch_gemv_b<BB, SYM>(a, st);
        LQ_B(1) LQ_B(2) LQ_B(3) LQ_B(4) LQ_B(5) LQ_B(6) LQ_B(7) LQ_B(8)
        LQ_B(9) LQ_B(10) LQ_B(11) LQ_B(12) LQ_B(13) LQ_B(14) LQ_B(15) LQ_B(16)
#undef LQ_B
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w4a16_gemv(const W4Args &a, hipStream_t st) {
    return a.symmetric ? launch_gemv_s<true>(a, st) : launch_gemv_s<false>(a, st);
}

}  // namespace lq
