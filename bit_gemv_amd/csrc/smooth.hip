// smooth.hip -- SmoothQuant migration strength and dynamic per-token INT8.
//
// "3.6 Quantization" (LLM learning path), section "SmoothQuant": for
// Y = X W with X[T][C_in], every positive s gives
// Y = (X diag(s)^-1)(diag(s) W); the method picks
// s_j = max_t |X_tj|^alpha / max |W_j|^(1 - alpha), where W_j is the weight
// row that multiplies input channel j (a column of our W[n][k]). Its code
// block then quantizes X / s per token and W * s per output channel to INT8.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// |v| of 8 bf16 values (one 16-byte word) folded into running maxima.
LQ_DEVICE void max8(float *m, const u32x4 v) {
    m[0] = fmaxf(m[0], fabsf(bf16_lo(v.x))); m[1] = fmaxf(m[1], fabsf(bf16_hi(v.x)));
    m[2] = fmaxf(m[2], fabsf(bf16_lo(v.y))); m[3] = fmaxf(m[3], fabsf(bf16_hi(v.y)));
    m[4] = fmaxf(m[4], fabsf(bf16_lo(v.z))); m[5] = fmaxf(m[5], fabsf(bf16_hi(v.z)));
    m[6] = fmaxf(m[6], fabsf(bf16_lo(v.w))); m[7] = fmaxf(m[7], fabsf(bf16_hi(v.w)));
}

// Column maxima of |W| over rows, folded into s[] with atomicMax on the
// bit patterns (non-negative floats order like their bits, and max is exact
// and order-free, so the result is deterministic). Block: 512 columns (a
// wave's 64 lanes x 8) x kColRows rows, the 4 waves taking every 4th row
// with 8 rows' loads in flight per lane; the waves' maxima meet in LDS, so
// each block issues one atomic per column, 64 consecutive columns per wave
// instruction. Measured on MI355X (8192 x 8192 bf16): 64-row tiles take
// 23.7 us, 128-row tiles 28.5 us (half the blocks); blocks owning whole
// 2048-column strips with the atomics straight from registers (8 columns a
// lane, 16 cache lines per instruction) were 1.2-2x slower.
constexpr int kColRows = 64;
constexpr int64_t kMaxGridY = 65535;  // hardware limit of a grid's y extent

__global__ __launch_bounds__(256) void colmax_kernel(const uint16_t *__restrict__ w, int64_t n, int64_t k,
                                                      uint32_t *__restrict__ acc) {
    __shared__ float red[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 512 + lane * 8;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // row tiles blockIdx.y, + gridDim.y, ... (the grid's y extent is capped)
    for (int64_t r0 = (int64_t)blockIdx.y * kColRows; col < k && r0 < n; r0 += (int64_t)gridDim.y * kColRows) {
        const int64_t r1 = r0 + kColRows < n ? r0 + kColRows : n;
        for (int64_t r = r0 + wave; r < r1; r += 32) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t rr = r + 4 * u;
                v[u] = rr < r1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w + rr * k + col))
                               : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) max8(m, v[u]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = threadIdx.x + 256 * h;
        const float v = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        if ((int64_t)blockIdx.x * 512 + c < k) atomicMax(acc + (int64_t)blockIdx.x * 512 + c, __float_as_uint(v));
    }
}

// Column maxima of |X| (32 columns per block: 4 lanes x 8 columns, 64 row
// phases with 8 rows' loads in flight, reduced through LDS), then
// s = f(ax, aw) with aw read from s[].
__global__ __launch_bounds__(256) void smooth_finalize_kernel(const uint16_t *__restrict__ x, int64_t t,
                                                               int64_t k, float alpha,
                                                               float *__restrict__ s) {
    __shared__ float red[64][33];
    const int cl = threadIdx.x & 3, ph = threadIdx.x >> 2;
    const int64_t col = (int64_t)blockIdx.x * 32 + cl * 8;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t r = ph; r < t; r += 512) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t rr = r + 64 * u;
            v[u] = rr < t ? *reinterpret_cast<const u32x4 *>(x + rr * k + col) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) max8(m, v[u]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[ph][cl * 8 + i] = m[i];
    __syncthreads();
    if (threadIdx.x < 32) {
        float ax = red[0][threadIdx.x];
        for (int p = 1; p < 64; ++p) ax = fmaxf(ax, red[p][threadIdx.x]);
        const int64_t j = (int64_t)blockIdx.x * 32 + threadIdx.x;
        float aw = s[j];  // the column max of |W| left by colmax_kernel
        const float a = ax < kFloor ? kFloor : ax;
        const float b = aw < kFloor ? kFloor : aw;
        float r;
        if (alpha == 0.5f)
            r = sqrtf(a) / sqrtf(b);
        else
            r = powf(a, alpha) / powf(b, 1.0f - alpha);
        s[j] = r;
    }
}

hipError_t launch_smooth_scale(const SmoothArgs &a, hipStream_t st) {
    uint32_t *acc = reinterpret_cast<uint32_t *>(a.s);
    hipLaunchKernelGGL(zero_u32_kernel, dim3((uint32_t)((a.k + 255) / 256)), dim3(256), 0, st, acc, a.k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = (a.n + kColRows - 1) / kColRows;
    dim3 grid((uint32_t)((a.k + 511) / 512), (uint32_t)(tiles < kMaxGridY ? tiles : kMaxGridY));
    hipLaunchKernelGGL(colmax_kernel, grid, dim3(256), 0, st, a.w, a.n, a.k, acc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(smooth_finalize_kernel, dim3((uint32_t)(a.k / 32)), dim3(256), 0, st, a.x, a.t, a.k,
                       a.alpha, a.s);
    return hipGetLastError();
}

// Per-token INT8: one block of TPB lanes per token. The row is read in
// chunks of kTokLoads * TPB * 8 elements, each lane issuing its kTokLoads
// 16-byte loads (and the matching smoothing factors) before any arithmetic;
// the quotients
// X / s of the chunk stay in registers. Maximum over every chunk, then codes
// from the chunk still in registers and from re-reads of the others, so a
// token of up to one chunk is read once. Measured on MI355X (512 x 8192
// with smoothing, X cold in HBM, calls replayed from a graph): 8.5 us, where
// one dependent load per lane at a time and the row read twice took 10.2 us.
constexpr int kTokLoads = 4;

// Quotients x / smooth (IEEE division, as the definition) of elements
// c0 + 8 t + 8 TPB i .. + 7 of the row; lanes past k produce zeros. FULL:
// k is a whole number of chunks, so no lane is past k. NT: the row is one
// chunk, read exactly once, so X comes with the streaming (non-temporal)
// hint; rows of several chunks read the earlier ones again and keep the
// default policy.
template <int TPB, bool SM, bool FULL, bool NT>
LQ_DEVICE void token_chunk(const uint16_t *__restrict__ xr, const float *__restrict__ smooth, int64_t k, int64_t c0,
                           int t, float f[kTokLoads][8]) {
    u32x4 v[kTokLoads];
    f32x4 d[kTokLoads][2];
#pragma unroll
    for (int i = 0; i < kTokLoads; ++i) {
        const int64_t e = c0 + t * 8 + 8 * TPB * i;
        const bool in = FULL || e < k;
        const u32x4 *p = reinterpret_cast<const u32x4 *>(xr + e);
        v[i] = !in ? u32x4{0u, 0u, 0u, 0u} : NT ? __builtin_nontemporal_load(p) : *p;
        if (SM) {
            const f32x4 one = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
            d[i][0] = in ? *reinterpret_cast<const f32x4 *>(smooth + e) : one;
            d[i][1] = in ? *reinterpret_cast<const f32x4 *>(smooth + e + 4) : one;
        }
    }
#pragma unroll
    for (int i = 0; i < kTokLoads; ++i) {
        f[i][0] = bf16_lo(v[i].x); f[i][1] = bf16_hi(v[i].x);
        f[i][2] = bf16_lo(v[i].y); f[i][3] = bf16_hi(v[i].y);
        f[i][4] = bf16_lo(v[i].z); f[i][5] = bf16_hi(v[i].z);
        f[i][6] = bf16_lo(v[i].w); f[i][7] = bf16_hi(v[i].w);
        if (SM) {
            f[i][0] /= d[i][0].x; f[i][1] /= d[i][0].y; f[i][2] /= d[i][0].z; f[i][3] /= d[i][0].w;
            f[i][4] /= d[i][1].x; f[i][5] /= d[i][1].y; f[i][6] /= d[i][1].z; f[i][7] /= d[i][1].w;
        }
    }
}

template <int TPB, bool SM, bool ONE, bool FULL>
__global__ __launch_bounds__(TPB) void token_quant_kernel(const uint16_t *__restrict__ x, int64_t k,
                                                           const float *__restrict__ smooth,
                                                           int8_t *__restrict__ qx, float *__restrict__ sx) {
    constexpr int kWaves = TPB / 64;
    constexpr int64_t kTokChunk = (int64_t)kTokLoads * TPB * 8;
    __shared__ float red[kWaves];
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * k;
    const int t = threadIdx.x;
    const int64_t nch = ONE ? 1 : (k + kTokChunk - 1) / kTokChunk;
    float f[kTokLoads][8];
    float a = 0.0f;
    for (int64_t ch = 0; ch < nch; ++ch) {
        token_chunk<TPB, SM, FULL, ONE>(xr, smooth, k, ch * kTokChunk, t, f);
#pragma unroll
        for (int i = 0; i < kTokLoads; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[i][j]));  // zeros past k change nothing
    }
    a = team_max<64>(a);
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) a = fmaxf(a, red[i]);
    const float am = a < kFloor ? kFloor : a;
    const float s = am / 127.0f;
    // X' / s through div_rn with y = RN(1 / s), once per token. It is the
    // IEEE quotient here: |X'| <= am = 127 s (finite), s >= 1e-8 / 127 and
    // y <= 1.3e10 are normal, and a quotient of magnitude 1/2 or more has
    // |X'| >= s / 2, so its residuals are normal as well; smaller quotients
    // round to 0 under either division.
    const float y = 1.0f / s;
    // the last chunk is still in f; the others are read again
    for (int64_t ch = nch - 1; ch >= 0; --ch) {
        if (ch != nch - 1) token_chunk<TPB, SM, FULL, ONE>(xr, smooth, k, ch * kTokChunk, t, f);
#pragma unroll
        for (int i = 0; i < kTokLoads; ++i) {
            const int64_t e = ch * kTokChunk + t * 8 + 8 * TPB * i;
            if (!FULL && e >= k) continue;
            // Rounding, clamp and byte in one add. The clamp never binds:
            // |X'| <= am and s = RN(am / 127) >= (am / 127)(1 - 2^-24), so
            // |RN(X' / s)| <= 127 (1 + 2^-23) and rounds to at most 127.
            // Floats in [2^23, 2^24) are the integers, so adding 2^23 + 256
            // (even) rounds the quotient to an integer with ties to even,
            // as rintf does, and leaves 256 + round(q), in 129 .. 383, in the
            // low mantissa bits: its low byte is the two's-complement byte
            // of round(q). Three byte permutes pack four of them.
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = __float_as_uint(div_rn(f[i][j], s, y) + 8388864.0f);
            const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(w[3], w[2], 0x0C0C0400u),
                                                      __builtin_amdgcn_perm(w[1], w[0], 0x0C0C0400u), 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(w[7], w[6], 0x0C0C0400u),
                                                      __builtin_amdgcn_perm(w[5], w[4], 0x0C0C0400u), 0x05040100u);
            // codes are written once: streaming stores (with the streaming
            // loads of one-chunk rows, 512 x 8192: 6.28-6.37 -> 5.83-5.90 us)
            __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2 *>(qx + row * k + e));
        }
    }
    if (t == 0) sx[row] = s;
}

template <int TPB>
static hipError_t launch_token_quant(const TokenQuantArgs &a, hipStream_t st) {
    constexpr int64_t kChunkK = (int64_t)kTokLoads * TPB * 8;
    const bool one = a.k <= kChunkK;
    // whole chunks: no lane past k, so the loads and stores need no guard
    // (512 x 8192 with smoothing: 7.7 -> 6.8 us)
    const bool full = a.k % kChunkK == 0;
#define LQ_TQ(SM, ONE, FULL)                                                                                    \
    if ((a.smooth != nullptr) == SM && one == ONE && full == FULL) {                                            \
        hipLaunchKernelGGL((token_quant_kernel<TPB, SM, ONE, FULL>), dim3((uint32_t)a.t), dim3(TPB), 0, st, a.x, \
                           a.k, a.smooth, a.qx, a.sx);                                                          \
        return hipGetLastError();                                                                               \
    }
    LQ_TQ(true, true, true) LQ_TQ(true, false, true) LQ_TQ(false, true, true) LQ_TQ(false, false, true)
    LQ_TQ(true, true, false) LQ_TQ(true, false, false) LQ_TQ(false, true, false) LQ_TQ(false, false, false)
#undef LQ_TQ
    return hipErrorInvalidValue;
}

// Lanes per token (measured, 512 tokens): 256 up to k = 8192, where larger
// blocks leave a CU room for one block only; 512 and 1024 lanes on wider
// rows (k = 8320: 9.8 against 12.9 us; k = 28672: 24.8 against 30.1 us).
hipError_t launch_quant_per_token(const TokenQuantArgs &a, hipStream_t st) {
    if (a.k <= 8192) return launch_token_quant<256>(a, st);
    if (a.k <= 16384) return launch_token_quant<512>(a, st);
    return launch_token_quant<1024>(a, st);
}

}  // namespace lq
