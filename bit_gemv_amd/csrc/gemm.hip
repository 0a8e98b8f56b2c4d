// gemm.hip -- W4A16 prefill GEMM on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Definition ("LLM quantization deep dive", rainlib.com, W4A16 and the
// prefill/decode split; "3.6 Quantization": weight-only quantization does not
// speed up compute-bound prefill, the product still runs on 16-bit operands):
//   Y[m][n] = sum_j X[m][j] (q[n][j] - z[n][j/G]) s[n][j/G].
// Prefill is compute-bound, so the product runs on the matrix cores with
// operands that are exact in bf16:
//  * weight operand 128 + q: a nibble ORed into the mantissa of bf16 128;
//  * per 128-wide group g, the tile D_g = sum_{j in g} X (128 + q) comes out
//    of four MFMAs into a fresh accumulator, and so does the activation sum
//    X_g = sum_{j in g} X (an MFMA against a bf16 ones operand, which lands in
//    the same lane layout as D_g);
//  * the fp32 correction acc += s (D_g - (128 + z) X_g) applies scale and
//    zero point exactly once per group; no weight is ever rounded to bf16.
// Tiles: a block of 4 waves computes 128 x 128 outputs (2 x 2 waves of
// 64 x 64 = 4 x 4 MFMA tiles of 16 x 16). Per group the block stages the
// 128 x 128 activation tile in LDS (double-buffered, padded rows); each wave
// loads its own code words from HBM (one 16-byte load per lane per 16
// columns) and unpacks them in registers.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, GK = 128;  // block tile and group width
constexpr int LDS_ROW = GK + 8;                // padded row (bf16): 272 bytes
constexpr uint32_t kNibPair = 0x000F000Fu;
constexpr uint32_t kMagicPair = 0x43004300u;   // bf16 pair (128, 128)
constexpr uint32_t kOnePair = 0x3F803F80u;     // bf16 pair (1, 1)

// Code word (element i at bits 4i..4i+3) -> 4 bf16 pairs (128 + c_2i,
// 128 + c_2i+1), i.e. natural k order: byte i of the word gives the low
// half, byte i of the word shifted right by 4 gives the high half.
LQ_DEVICE u32x4 unpack_natural(uint32_t w, uint32_t magic) {
    const uint32_t w4 = w >> 4;
    u32x4 p;
    p.x = (__builtin_amdgcn_perm(w4, w, 0x0C040C00u) & kNibPair) | magic;
    p.y = (__builtin_amdgcn_perm(w4, w, 0x0C050C01u) & kNibPair) | magic;
    p.z = (__builtin_amdgcn_perm(w4, w, 0x0C060C02u) & kNibPair) | magic;
    p.w = (__builtin_amdgcn_perm(w4, w, 0x0C070C03u) & kNibPair) | magic;
    return p;
}

template <bool SYM>
__global__ __launch_bounds__(256) void gemm_w4_kernel(const uint16_t *__restrict__ x, int m, int n, int k,
                                                       const uint8_t *__restrict__ codes,
                                                       const float *__restrict__ scales,
                                                       const float *__restrict__ zeros, int group,
                                                       float *__restrict__ y) {
    __shared__ uint16_t a_lds[2][BM][LDS_ROW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int l16 = lane & 15, kq = lane >> 4;
    const int ng = k / group;
    const int ngroups = k / GK;

    // activation rows of this block; rows past m read zeros
    const int rows_m = min(BM, m - m0);
    const auto rx = make_rsrc(x + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k * 2);
    // code rows of this block; rows past n read zeros
    const int rows_n = min(BN, n - n0);
    const uint32_t row_bytes = (uint32_t)k / 2;
    const auto rc = make_rsrc(codes + (int64_t)n0 * row_bytes, (uint32_t)rows_n * row_bytes);
    const auto rs = make_rsrc(scales + (int64_t)n0 * ng, (uint32_t)rows_n * ng * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)n0 * ng, SYM ? 0u : (uint32_t)rows_n * ng * 4);

    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagicPair));
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{kOnePair, kOnePair, kOnePair, kOnePair});

    // staging: thread t moves 16-byte chunks t + 256 i (i = 0..7) of the
    // 128 x 128 activation tile: row t / 16 + 16 i, columns 8 (t % 16) + [0, 8)
    const int st_row = tid >> 4, st_col = (tid & 15) * 8;
    u32x4 stage[8];
    auto load_stage = [&](int g) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            stage[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, ((uint32_t)(st_row + 16 * i) * (uint32_t)k + g * GK + st_col) * 2, 0, 0);
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4 *>(&a_lds[buf][st_row + 16 * i][st_col]) = stage[i];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int g = 0; g < ngroups; ++g) {
        const int buf = g & 1;
        if (g + 1 < ngroups) load_stage(g + 1);  // next group's activations, in flight during this one

        // this wave's code words: column wn*64 + nt*16 + l16, k quarter kq of the group
        u32x4 cw[4];
        float sc[4], zc[4];
        const int gi = (g * GK) / group;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const uint32_t col = wn * 64 + nt * 16 + l16;
            // cached: the same code words are read by every m-block
            cw[nt] = __builtin_amdgcn_raw_buffer_load_b128(rc, col * row_bytes + g * (GK / 2) + kq * 16, 0, 0);
            sc[nt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (col * ng + gi) * 4, 0, 0));
            zc[nt] = SYM ? 0.0f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, (col * ng + gi) * 4, 0, 0));
        }

        f32x4 d[4][4], xg[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            xg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) d[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // MFMA k-step: lane k quarter kq, word j -> k = 32 kq + 8 j + [0, 8)
            bf16x8_t bop[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t w = j == 0 ? cw[nt].x : j == 1 ? cw[nt].y : j == 2 ? cw[nt].z : cw[nt].w;
                bop[nt] = __builtin_bit_cast(bf16x8_t, unpack_natural(w, magic));
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8_t aop = *reinterpret_cast<const bf16x8_t *>(
                    &a_lds[buf][wm * 64 + mt * 16 + l16][kq * 32 + j * 8]);
                xg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, ones, xg[mt], 0, 0, 0);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    d[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[nt], d[mt][nt], 0, 0, 0);
            }
        }
        // acc += s (D_g - (128 + z) X_g); lane holds rows 4 kq + v, column l16
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const float c = SYM ? 136.0f : 128.0f + zc[nt];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[mt][nt][v] = __builtin_fmaf(sc[nt], __builtin_fmaf(-c, xg[mt][v], d[mt][nt][v]),
                                                    acc[mt][nt][v]);
        }
        if (g + 1 < ngroups) {
            store_stage(buf ^ 1);
            __syncthreads();
        }
    }
    // epilogue: lane holds Y[row 4 kq + v][col l16] of each 16 x 16 tile
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + mt * 16 + kq * 4 + v;
                const int col = n0 + wn * 64 + nt * 16 + l16;
                if (row < m && col < n) y[(int64_t)row * n + col] = acc[mt][nt][v];
            }
}

}  // namespace

hipError_t launch_w4a16_gemm(const W4Args &a, hipStream_t st) {
    dim3 grid((uint32_t)((a.n + BN - 1) / BN), (uint32_t)((a.m + BM - 1) / BM));
    if (a.symmetric)
        hipLaunchKernelGGL(gemm_w4_kernel<true>, grid, dim3(256), 0, st, a.x, (int)a.m, (int)a.n, (int)a.k, a.codes,
                           a.scales, a.zeros, (int)a.group, a.y);
    else
        hipLaunchKernelGGL(gemm_w4_kernel<false>, grid, dim3(256), 0, st, a.x, (int)a.m, (int)a.n, (int)a.k,
                           a.codes, a.scales, a.zeros, (int)a.group, a.y);
    return hipGetLastError();
}

}  // namespace lq
