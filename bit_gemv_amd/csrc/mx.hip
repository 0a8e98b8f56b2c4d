// mx.hip -- MXFP4 weights on gfx950: the block quantizer and the decode GEMV
// with 16-bit activations.
//
// Format ("3.6 Quantization", number-format table: FP4 E2M1 elements with
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, in blocks of 32 sharing one 8-bit
// power-of-two scale, E8M0, as in the OCP Microscaling standard; "Granularity":
// one scale per block of 32; compendium "Microscaling (MX) formats": a block
// shares an exponent, each element keeps its own bits). Readings where the
// pages leave a step open:
//  - a block is 32 consecutive elements of a row along k;
//  - the shared scale 2^e is the smallest power of two with amax <= 6 * 2^e
//    (the absmax rule restricted to powers of two: no element clips), e
//    clamped to [-127, 127], stored as the E8M0 byte e + 127 (an all-zero
//    block stores 0);
//  - an element is x / 2^e rounded to the nearest E2M1 magnitude, ties to
//    the even encoding, with the sign of x; a zero magnitude is stored +0;
//  - two codes per byte, element 2j in the low nibble; the nibble is
//    sign << 3 | exponent << 1 | mantissa.
// The GEMV: y[b][r] = sum_j x[b][j] * E2M1(c[r][j]) * 2^e[r][j/32].
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

// e = smallest integer with amax <= 6 * 2^e = 1.5 * 2^(e + 2), from the bits
// of amax: amax = f * 2^E with f in [1, 2) gives e = E - 2 + (f > 1.5).
LQ_DEVICE int mx_exponent(float amax) {
    // zero and subnormal amax (below 2^-126) land below the E8M0 range: -127
    const uint32_t u = __float_as_uint(amax);
    if ((u >> 23) == 0) return -127;
    const int e = (int)(u >> 23) - 127 - 2 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Codes of 8 elements (one 16-byte chunk of bf16) with the block exponent e:
// element j's nibble at bits 4j..4j+3. v_cvt_scalef32_pk_fp4_bf16 computes
// x / 2^e rounded to the nearest E2M1 value, ties to the even encoding, for
// two bf16 at a time -- the rounding read from the pages, checked on the
// device for every finite bf16 value at scales 2^-127 .. 2^127. The scale
// operand is the E8M0 byte in the fp32 exponent field (the byte 0, 0.0f,
// acts as 2^-127). The conversion keeps the sign of a value that rounds to
// magnitude 0 (code 8, -0); such codes are turned into +0 afterwards.
LQ_DEVICE uint32_t e2m1_codes8(const u32x4 v, int e) {
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
    // each pair into byte 0 of a zero word (the form checked on the device),
    // then shifted into place. (The words are copied out of the vector
    // first: a bit-cast of a vector element itself read element 0.)
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t pair = __builtin_bit_cast(bf16x2_t, words[i]);
        c |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, pair, scale, 0) & 0xFFu) << (8 * i);
    }
    // keep the sign bit of a nibble only where its magnitude is nonzero
    const uint32_t mag = c & 0x77777777u;
    const uint32_t nz = (mag | (mag >> 1) | (mag >> 2)) & 0x11111111u;
    return mag | (c & (nz << 3));
}

// A lane quantizes kMxChunks chunks of 8 elements (16 bytes of bf16), all
// loads issued first; 4 consecutive lanes of a chunk slice form a block of
// 32 and share its maximum through two DPP steps. The matrix is flattened:
// k is a multiple of 32, so blocks never span rows and block b covers
// elements [32 b, 32 b + 32), code bytes [16 b, 16 b + 16) and scale byte b.
constexpr int kMxChunks = 4;

// FULL: the block's chunks all exist (every block but the last), so its
// loads and stores need no guard.
template <bool FULL>
LQ_DEVICE void mx_quant_body(const uint16_t *__restrict__ w, int64_t total8, uint8_t *__restrict__ codes,
                             uint8_t *__restrict__ scales) {
    const int64_t base = (int64_t)blockIdx.x * (256 * kMxChunks) + threadIdx.x;
    u32x4 v[kMxChunks];
#pragma unroll
    for (int c = 0; c < kMxChunks; ++c) {
        const int64_t i = base + 256 * c;
        // lanes past the end take part in the 4-lane maximum with zeros
        v[c] = FULL || i < total8 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w) + i)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < kMxChunks; ++c) {
        const int64_t i = base + 256 * c;
        const uint32_t words[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(bf16_lo(words[j])), fabsf(bf16_hi(words[j]))));
        // maximum over the block's 4 lanes (aligned quads of the wave)
        a = fmaxf(a, dpp_move<kDppXor1>(a));
        a = fmaxf(a, dpp_move<kDppXor2>(a));
        const int e = mx_exponent(a);
        const uint32_t packed = e2m1_codes8(v[c], e);
        if (FULL || i < total8) {
            // streaming code stores (written once): 70B stack 5.87-5.90 ->
            // 5.56-5.59 ms; the hint on the scale bytes as well measured slower
            __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(codes) + i);
            if ((threadIdx.x & 3) == 0) scales[i >> 2] = (uint8_t)(e + 127);
        }
    }
}

__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t *__restrict__ w, int64_t total8,
                                                       uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    if ((int64_t)(blockIdx.x + 1) * (256 * kMxChunks) <= total8)
        mx_quant_body<true>(w, total8, codes, scales);
    else
        mx_quant_body<false>(w, total8, codes, scales);
}

// ---------------------------------------------------------------------------
// GEMV, batch 1..16 (VALU). A lane owns 32 consecutive k of a row -- one
// 16-byte code load and exactly one MX block -- so a wave load covers 2048 k.
// v_cvt_scalef32_pk_bf16_fp4 turns each code byte into the exact bf16 pair
// (E2M1 of the low nibble, E2M1 of the high nibble), which is the natural k
// order of the activation word holding the same two k; v_dot2_f32_bf16
// multiplies them (products exact in fp32) and the block's 2^e scales the
// lane's sum once, exactly, in fp32. Block layout as the INT4 kernel: 4
// waves split the chunks of k (ks_count ways) and the block's rows; the
// 64 scale bytes of each of a wave's rows per chunk come from one 16-byte
// load per lane (lanes 0 .. 4 RW - 1), passed through the wave's LDS slice.
// ---------------------------------------------------------------------------
constexpr int kMxChunk = 2048;

// 2^(s - 127) for an E8M0 byte s (s = 0 is the subnormal 2^-127)
LQ_DEVICE float e8m0_value(uint32_t s) { return __uint_as_float(s ? s << 23 : 0x00400000u); }

template <int B, int RW>
__global__ __launch_bounds__(256) void mx_gemv_kernel(const uint16_t *__restrict__ x, int bsz,
                                                      const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int n, int k,
                                                      int ks_count, float *__restrict__ y) {
    static_assert(RW == 4 || RW == 8, "rows per wave: 4 or 8");
    static_assert(RW * B <= 64, "the final sum gives one output per lane");
    __shared__ float red[4][B][RW];
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[4][RW][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks_log = ks_count == 4 ? 2 : ks_count - 1;
    const int ks = wave & (ks_count - 1);
    const int rs = wave >> ks_log;
    const int row0 = (blockIdx.x * (4 >> ks_log) + rs) * RW;
    const int nblk = k / 32;
    const int nchunks = (k + kMxChunk - 1) / kMxChunk;
    const int rows_here = row0 < n ? min(RW, n - row0) : 0;
    const uint32_t row_bytes = (uint32_t)k / 2;
    const auto rc = make_rsrc(codes + (int64_t)row0 * row_bytes, (uint32_t)rows_here * row_bytes);
    const auto rsc = make_rsrc(scales + (int64_t)row0 * nblk, (uint32_t)(rows_here * nblk));

    float acc[B][RW];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[b][r] = 0.0f;

    // batch rows are taken BP at a time: a lane's 32 activations of one batch
    // row are 16 registers, so all 16 rows at once would not fit with the codes
    constexpr int BP = B < 4 ? B : 4;
    for (int c = ks; c < nchunks; c += ks_count) {
        const int k0 = c * kMxChunk + lane * 32;
        const bool kv = k0 < k;
        const uint32_t xo = kv ? (uint32_t)k0 * 2 : kOutOfRange;
        auto load_x = [&](int b0, u32x4 (&xv)[BP][4]) {
#pragma unroll
            for (int b = 0; b < BP; ++b) {
                const auto rx = make_rsrc(x + (int64_t)(b0 + b) * k, b0 + b < bsz ? (uint32_t)k * 2 : 0u);
#pragma unroll
                for (int j = 0; j < 4; ++j) xv[b][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * j, 0, 0);
            }
        };
        u32x4 xv[BP][4];
        load_x(0, xv);
        const uint32_t co = kv ? (uint32_t)k0 / 2 : kOutOfRange;
        u32x4 cw[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r)
            cw[r] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + r * row_bytes, 0, kNonTemporal);
        // scale bytes: lane L < 4 RW loads row L / 4, bytes 16 (L % 4) .. + 15 of the chunk
        const int sr = lane >> 2, sq = lane & 3;
        const int sb = c * (kMxChunk / 32) + 16 * sq;
        const uint32_t so = sr < RW && sb < nblk ? (uint32_t)(sr * nblk + sb) : kOutOfRange;
        const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rsc, so, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (sr < RW) *reinterpret_cast<u32x4 *>(&sc_lds[wave][sr][16 * sq]) = sv;
        // one wave writes and reads its slice: LDS runs them in order; keep
        // the compiler from moving the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float sc[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) sc[r] = kv ? e8m0_value(sc_lds[wave][r][lane]) : 0.0f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int b0 = 0; b0 < B; b0 += BP) {
            if (b0 > 0) {
                // keep the next rows' loads (and registers) out of the previous pass
                __builtin_amdgcn_sched_barrier(0);
                load_x(b0, xv);
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const uint32_t cwv[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
                uint32_t p[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwv[q], 1.0f, 0));
                    p[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwv[q], 1.0f, 1));
                    p[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwv[q], 1.0f, 2));
                    p[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwv[q], 1.0f, 3));
                }
#pragma unroll
                for (int b = 0; b < BP; ++b) {
                    float d = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        d = dot2_bf16(p[4 * j + 0], xv[b][j].x, d);
                        d = dot2_bf16(p[4 * j + 1], xv[b][j].y, d);
                        d = dot2_bf16(p[4 * j + 2], xv[b][j].z, d);
                        d = dot2_bf16(p[4 * j + 3], xv[b][j].w, d);
                    }
                    acc[b0 + b][r] = __builtin_fmaf(d, sc[r], acc[b0 + b][r]);
                }
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

template <int B, int RW>
hipError_t launch_mx_rw(const MxArgs &a, hipStream_t st, int ks_count) {
    const int rows_per_block = (4 / ks_count) * RW;
    const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((mx_gemv_kernel<B, RW>), dim3((uint32_t)blocks), dim3(256), 0, st, a.x, (int)a.m, a.codes,
                       a.scales, (int)a.n, (int)a.k, ks_count, a.y);
    return hipGetLastError();
}

// Launch shape as the INT4 kernel (same code bytes per chunk): k split 4
// ways at 4..7 chunks a row, 2 ways at 2..3 or 8 and more; 8 rows a wave
// (batch up to 4) from 512 blocks, with the four-way split from more than
// 512 (measured at batch 1: the 70B shapes are at the best of ks x rows;
// 4096 x 11008 takes 7.35 us with 4 rows against 8.12 with 8).
template <int B>
hipError_t launch_mx(const MxArgs &a, hipStream_t st) {
    const int nchunks = (int)((a.k + kMxChunk - 1) / kMxChunk);
    const int ks = nchunks >= 8 ? 2 : nchunks >= 4 ? 4 : nchunks >= 2 ? 2 : 1;
    const int64_t blocks8 = (a.n + (4 / ks) * 8 - 1) / ((4 / ks) * 8);
    if constexpr (B <= 4) {  // 8 rows at larger batches would not fit the registers
        if (ks == 4 ? blocks8 > 512 : blocks8 >= 512) return launch_mx_rw<B, 8>(a, st, ks);
    }
    return launch_mx_rw<B, 4>(a, st, ks);
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales,
                              hipStream_t st) {
    const int64_t total8 = n * k / 8;
    hipLaunchKernelGGL(mx_quant_kernel, dim3((uint32_t)((total8 + 256 * kMxChunks - 1) / (256 * kMxChunks))), dim3(256),
                       0, st, w, total8, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_gemv(const MxArgs &a, hipStream_t st) {
    // batch 4..16 on large matrices: the shared-stage kernel of gemv_shared.hip
    if (shared_gemv_pays(WeightFormat::kMx, a.m, a.n, a.k)) {
        const SharedGemvArgs sa{a.x, a.m, a.codes, a.scales, nullptr, a.n, a.k, 0, 32, a.y};
        return launch_shared_gemv(WeightFormat::kMx, sa, st);
    }
    switch (a.m) {
        case 1: return launch_mx<1>(a, st);
        case 2: return launch_mx<2>(a, st);
        case 3: return launch_mx<3>(a, st);
        case 4: return launch_mx<4>(a, st);
        default:
            if (a.m <= 8) return launch_mx<8>(a, st);
            if (a.m <= 16) return launch_mx<16>(a, st);
            return hipErrorInvalidValue;
    }
}

}  // namespace lq
