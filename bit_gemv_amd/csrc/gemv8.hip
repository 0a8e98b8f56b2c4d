// gemv8.hip -- W8A16 decode GEMV for gfx950 (batch 1..16), a VALU
// (v_dot2_f32_bf16) kernel.
//
// Definition ("LLM quantization deep dive", rainlib.com: the W/A/KV notation
// names W8A16 -- 8-bit weights, 16-bit activations -- and, as for W4A16, the
// codes are dequantized inside the kernel and multiplied with the 16-bit
// activations, accumulating at higher precision):
//   y[b][r] = sum_j x[b][j] * (q[r][j] - z[r][j/G]) * s[r][j/G].
// At small batch the product is bound by the code bytes streamed from HBM,
// one byte per weight here. Design:
//
//  * A code byte u (0..255) has at most 8 significant bits, so bf16 holds it
//    exactly: v_cvt_f32_ubyte{0..3} gives its fp32 value and the upper halves
//    of two such floats form a bf16 pair in natural k order, which meets the
//    activation word holding the same two k. Products with bf16 activations
//    are exact in fp32. (Unlike INT4, a byte does not fit the 7-bit mantissa
//    of a bf16 constant, so the OR-into-mantissa unpacking does not apply.)
//  * Symmetric codes are int8: xor 0x80 turns q into u = q + 128. The zero
//    point (asymmetric) or the offset 128 (symmetric) is folded into a
//    per-group correction: sum x (q - z) s = s (sum x u - c sum x), c = z or
//    128, with sum x formed once per activation segment.
//  * A lane owns 16 consecutive k of a row, one 16-byte load, so a wave-wide
//    load covers 1024 k and a lane's k never straddle a group (groups are
//    multiples of 128).
// Block layout: 4 waves split the 1024-wide chunks of k (ks_count ways) and
// the block's rows (4 / ks_count row sets of RW rows). Per chunk a wave
// issues its activation loads (L2 hits), the 16-byte code loads of its RW
// rows and one 4-byte scale (and zero) load per lane covering RW rows x 8
// groups, then computes. Per-row partial sums stay in registers until one
// reduction inside the wave and one through LDS; no atomics, so results are
// deterministic. Batch 5..16 on large matrices goes to the shared-stage
// kernel of gemv_shared.hip instead.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

constexpr int kChunk8 = 1024;               // k covered by one wave-wide 16-byte load
constexpr uint32_t kOnesPair = 0x3F803F80u;  // bf16 pair (1, 1)

// Four code bytes u0..u3 -> bf16 pairs (u0, u1) and (u2, u3). The byte-wise
// integer-to-float conversions select v_cvt_f32_ubyte{0..3}; the upper half
// of an fp32 holding an integer below 256 is its exact bf16.
LQ_DEVICE void bytes_to_bf16(uint32_t w, uint32_t &p01, uint32_t &p23) {
    const float f0 = (float)(w & 0xFFu);
    const float f1 = (float)((w >> 8) & 0xFFu);
    const float f2 = (float)((w >> 16) & 0xFFu);
    const float f3 = (float)(w >> 24);
    p01 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    p23 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// B: batch rows the kernel is built for (bsz <= B are used; the rest read
// zeros and are not stored). RW: rows per wave (4 or 8).
template <int B, int RW, bool SYM>
__global__ __launch_bounds__(256) void gemv8_kernel(const uint16_t *__restrict__ x, int bsz,
                                                     const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ scales,
                                                     const float *__restrict__ zeros, int n, int k, int group,
                                                     int ks_count, float *__restrict__ y) {
    static_assert(RW == 4 || RW == 8, "rows per wave: 4 or 8");
    static_assert(RW * B <= 64, "the final sum gives one output per lane");
    __shared__ float red[4][B][RW];
    // per wave: [scale | zero][group within the chunk][row]
    __shared__ __attribute__((aligned(16))) float sz_lds[4][2][8][RW];
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) so the buffer resources below live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks_log = ks_count == 4 ? 2 : ks_count - 1;  // ks_count is 1, 2 or 4
    const int ks = wave & (ks_count - 1);
    const int rs = wave >> ks_log;
    const int row0 = (blockIdx.x * (4 >> ks_log) + rs) * RW;
    const int ng = k / group;
    const int nchunks = (k + kChunk8 - 1) / kChunk8;
    const int rows_here = row0 < n ? min(RW, n - row0) : 0;
    const uint32_t row_bytes = (uint32_t)k;
    // rows past n read zeros through these resources
    const auto rc = make_rsrc(codes + (int64_t)row0 * k, (uint32_t)rows_here * row_bytes);
    const auto rsc = make_rsrc(scales + (int64_t)row0 * ng, (uint32_t)(rows_here * ng) * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)row0 * ng, SYM ? 0u : (uint32_t)(rows_here * ng) * 4);
    // lane L loads the scale (and zero) of row L / 8, group L % 8 of the chunk
    const int sg_lane = lane & 7, sr_lane = lane >> 3;

    float acc[B][RW];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[b][r] = 0.0f;

    for (int c = ks; c < nchunks; c += ks_count) {
        const int k0 = c * kChunk8 + lane * 16;
        const bool kv = k0 < k;
        // all loads of the chunk first; nothing waits until all are issued
        u32x4 xv[B][2];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const auto rx = make_rsrc(x + (int64_t)b * k, b < bsz ? (uint32_t)k * 2 : 0u);
            const uint32_t xo = kv ? (uint32_t)k0 * 2 : kOutOfRange;
            xv[b][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
            xv[b][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, 0, 0);
        }
        const uint32_t co = kv ? (uint32_t)k0 : kOutOfRange;
        u32x4 cw[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r)
            cw[r] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + r * row_bytes, 0, kNonTemporal);
        // a 1024-wide chunk starting at a multiple of 128 touches at most 8 groups
        const int g_first = c * (kChunk8 / 128) * 128 / group;
        const int sg = g_first + sg_lane;
        const uint32_t so = sg < ng && sr_lane < RW ? (uint32_t)(sr_lane * ng + sg) * 4 : kOutOfRange;
        const float sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, so, 0, 0));
        const float zv = SYM ? 0.0f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, so, 0, 0));
        __builtin_amdgcn_sched_barrier(0);

        // transpose the scales (zeros) through the wave's LDS slice
        if (sr_lane < RW) {
            sz_lds[wave][0][sg_lane][sr_lane] = sv;
            if (!SYM) sz_lds[wave][1][sg_lane][sr_lane] = zv;
        }
        // writes and reads are one wave's: LDS runs them in order; keep the
        // compiler from moving the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int gl = kv ? k0 / group - g_first : 0;
        float sc[RW], cz[RW];
#pragma unroll
        for (int r4 = 0; r4 < RW; r4 += 4) {
            const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][0][gl][r4]);
            sc[r4] = s4.x; sc[r4 + 1] = s4.y; sc[r4 + 2] = s4.z; sc[r4 + 3] = s4.w;
            if (SYM) {
                cz[r4] = cz[r4 + 1] = cz[r4 + 2] = cz[r4 + 3] = 128.0f;
            } else {
                const f32x4 z4 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][1][gl][r4]);
                cz[r4] = z4.x; cz[r4 + 1] = z4.y; cz[r4 + 2] = z4.z; cz[r4 + 3] = z4.w;
            }
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) sc[r] = kv ? sc[r] : 0.0f;

        float xs[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float t = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                t = dot2_bf16(xv[b][h].x, kOnesPair, t);
                t = dot2_bf16(xv[b][h].y, kOnesPair, t);
                t = dot2_bf16(xv[b][h].z, kOnesPair, t);
                t = dot2_bf16(xv[b][h].w, kOnesPair, t);
            }
            xs[b] = t;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            u32x4 w = cw[r];
            if (SYM) w ^= 0x80808080u;
            uint32_t p[8];
            bytes_to_bf16(w.x, p[0], p[1]);
            bytes_to_bf16(w.y, p[2], p[3]);
            bytes_to_bf16(w.z, p[4], p[5]);
            bytes_to_bf16(w.w, p[6], p[7]);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float d = 0.0f;
                d = dot2_bf16(p[0], xv[b][0].x, d);
                d = dot2_bf16(p[1], xv[b][0].y, d);
                d = dot2_bf16(p[2], xv[b][0].z, d);
                d = dot2_bf16(p[3], xv[b][0].w, d);
                d = dot2_bf16(p[4], xv[b][1].x, d);
                d = dot2_bf16(p[5], xv[b][1].y, d);
                d = dot2_bf16(p[6], xv[b][1].z, d);
                d = dot2_bf16(p[7], xv[b][1].w, d);
                acc[b][r] = __builtin_fmaf(sc[r], __builtin_fmaf(-cz[r], xs[b], d), acc[b][r]);
            }
        }
    }
    constexpr int P = RW == 4 ? 2 : 3;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float v = reduce_rows<RW>(acc[b], lane);
        if ((lane & ((64 >> P) - 1)) == 0) red[wave][b][lane >> (6 - P)] = v;
    }
    __syncthreads();
    if (ks == 0 && lane < RW * B) {
        const int b = lane / RW, r = lane % RW;
        float v = 0.0f;
        for (int w = 0; w < ks_count; ++w) v += red[rs * ks_count + w][b][r];
        const int row = row0 + r;
        if (row < n && b < bsz) y[(int64_t)b * n + row] = v;
    }
}

template <int B, int RW, bool SYM>
static hipError_t launch8_rw(const WoArgs &a, hipStream_t st, int ks_count) {
    const int rows_per_block = (4 / ks_count) * RW;
    const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv8_kernel<B, RW, SYM>), dim3((uint32_t)blocks), dim3(256), 0, st, a.x, (int)a.m,
                       a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, ks_count, a.y);
    return hipGetLastError();
}

// Launch shape: four waves share k four ways at 4..7 chunks a row, two ways
// at 2..3 or 8 and more, not at all for one chunk; 8 rows a wave when that
// still leaves 512 blocks and the batch allows it. At batch 1..3 rows of 8
// and more chunks also split four ways: at batch 1 with 4 rows a wave below
// 16 chunks (measured on the 70B shapes, us per launch, two-way split ->
// four-way: 10240 x 8192 19.9 -> 16.4, 8192 x 8192 15.7 -> 13.5, 57344 x
// 8192 80.9 -> 74.4, 8192 x 28672 with 8 rows 43.4 -> 39.3), at batch 2 and
// 3 with 8 rows (batch 2: 22.6 -> 18.5, 16.4 -> 15.2, 85.2 -> 77.7,
// 46.5 -> 43.0; batch 3: 2-11 % faster).
template <int B, bool SYM>
static hipError_t launch8(const WoArgs &a, hipStream_t st) {
    const int nchunks = (int)((a.k + kChunk8 - 1) / kChunk8);
    if constexpr (B <= 3) {
        if (nchunks >= 8) {
            const bool tall = (a.n + 7) / 8 >= 512;
            const bool rw8 = tall && (B > 1 || nchunks >= 16);
            return rw8 ? launch8_rw<B, 8, SYM>(a, st, 4) : launch8_rw<B, 4, SYM>(a, st, 4);
        }
    }
    const int ks = nchunks >= 8 ? 2 : nchunks >= 4 ? 4 : nchunks >= 2 ? 2 : 1;
    const int64_t blocks8 = (a.n + (4 / ks) * 8 - 1) / ((4 / ks) * 8);
    if constexpr (B <= 8) {
        if (blocks8 >= 512) return launch8_rw<B, 8, SYM>(a, st, ks);
    }
    return launch8_rw<B, 4, SYM>(a, st, ks);
}

template <bool SYM>
static hipError_t launch8_s(const WoArgs &a, hipStream_t st) {
    switch (a.m) {
        case 1: return launch8<1, SYM>(a, st);
        case 2: return launch8<2, SYM>(a, st);
        case 3: return launch8<3, SYM>(a, st);
        case 4: return launch8<4, SYM>(a, st);
        default: return a.m <= 8 ? launch8<8, SYM>(a, st) : launch8<16, SYM>(a, st);
    }
}

hipError_t launch_w8a16_gemv(const WoArgs &a, hipStream_t st) {
    if (a.m < 1 || a.m > 16) return hipErrorInvalidValue;
    // batch 4..16 on large matrices: the shared-stage kernel of gemv_shared.hip
    if (shared_gemv_pays(WeightFormat::kInt8, a.m, a.n, a.k)) {
        const SharedGemvArgs sa{a.x, a.m, a.codes, a.scales, a.zeros, a.n, a.k, a.symmetric, a.group, a.y};
        return launch_shared_gemv(WeightFormat::kInt8, sa, st);
    }
    return a.symmetric ? launch8_s<true>(a, st) : launch8_s<false>(a, st);
}

}  // namespace lq
