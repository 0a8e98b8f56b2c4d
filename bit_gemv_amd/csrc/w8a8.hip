// w8a8.hip -- INT8 x INT8 GEMM with INT32 accumulation and fp32 rescale on
// gfx950 int8 MFMA (v_mfma_i32_16x16x64_i8).
//
// Definition (compendium "Quantization", activation quantization: INT8
// weights and activations multiplied with INT32 accumulation; "3.6
// Quantization" code block: one scale per token times one per output
// channel):
//   acc[m][n] = sum_j qx[m][j] qw[n][j]  (exact int32)
//   y[m][n]   = ((float) acc[m][n] * sx[m]) * sw[n]
// Both operands are K-contiguous, so a lane's 16-byte slice of a row is an
// MFMA operand fragment as loaded. A block of 4 waves computes 128 x 128
// outputs (2 x 2 waves of 64 x 64 = 4 x 4 tiles of 16 x 16); per 64-wide
// k-step it stages the 128 x 64 slices of qx and qw in LDS (double-buffered,
// rows padded to 80 bytes so fragment reads are bank-conflict-free).
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LROW = BK + 16;  // padded LDS row, bytes

__global__ __launch_bounds__(256) void w8a8_kernel(const int8_t *__restrict__ qx, const float *__restrict__ sx,
                                                    int m, const int8_t *__restrict__ qw,
                                                    const float *__restrict__ sw, int n, int k,
                                                    int32_t *__restrict__ accout, float *__restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t a_lds[2][BM * LROW];
    __shared__ __attribute__((aligned(16))) int8_t b_lds[2][BN * LROW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int l16 = lane & 15, kq = lane >> 4;

    const int rows_m = min(BM, m - m0), rows_n = min(BN, n - n0);
    const auto ra = make_rsrc(qx + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k);
    const auto rb = make_rsrc(qw + (int64_t)n0 * k, (uint32_t)rows_n * (uint32_t)k);

    // staging: each 128 x 64 slice is 512 chunks of 16 bytes; thread t moves
    // chunks t and t + 256 of each operand: row t / 4 (+ 64), column 16 (t % 4)
    const int st_row = tid >> 2, st_col = (tid & 3) * 16;
    u32x4 sa[2], sb[2];
    auto load_stage = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t off = (uint32_t)(st_row + 64 * i) * (uint32_t)k + ks * BK + st_col;
            sa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
            sb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, kNonTemporal);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4 *>(&a_lds[buf][(st_row + 64 * i) * LROW + st_col]) = sa[i];
            *reinterpret_cast<u32x4 *>(&b_lds[buf][(st_row + 64 * i) * LROW + st_col]) = sb[i];
        }
    };

    i32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nsteps = k / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int ks = 0; ks < nsteps; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nsteps) load_stage(ks + 1);
        // fragments: lane (row l16, k quarter kq) holds 16 consecutive bytes
        i32x4 af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            af[t] = *reinterpret_cast<const i32x4 *>(&a_lds[buf][(wm * 64 + t * 16 + l16) * LROW + kq * 16]);
            bf[t] = *reinterpret_cast<const i32x4 *>(&b_lds[buf][(wn * 64 + t * 16 + l16) * LROW + kq * 16]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        if (ks + 1 < nsteps) {
            store_stage(buf ^ 1);
            __syncthreads();
        }
    }
    // epilogue: lane holds acc[row 4 kq + v][col l16] of each tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + l16;
        const float swc = col < n ? sw[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + i * 16 + kq * 4 + v;
                if (row < m && col < n) {
                    const int32_t a = acc[i][j][v];
                    if (accout) accout[(int64_t)row * n + col] = a;
                    y[(int64_t)row * n + col] = ((float)a * sx[row]) * swc;
                }
            }
    }
}

}  // namespace

hipError_t launch_w8a8_gemm(const W8Args &a, hipStream_t st) {
    dim3 grid((uint32_t)((a.n + BN - 1) / BN), (uint32_t)((a.m + BM - 1) / BM));
    hipLaunchKernelGGL(w8a8_kernel, grid, dim3(256), 0, st, a.qx, a.sx, (int)a.m, a.qw, a.sw, (int)a.n, (int)a.k,
                       a.acc, a.y);
    return hipGetLastError();
}

}  // namespace lq
