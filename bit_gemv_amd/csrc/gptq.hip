// gptq.hip -- GPTQ error-compensated rounding on gfx950.
//
// Method ("3.6 Quantization", GPTQ section; "LLM quantization deep dive" and
// the PTQ concept page, GPTQ): per layer, minimise ||W X - W_hat X||^2 on
// calibration data by quantizing W one input column at a time and moving
// the columns not yet quantized to absorb each rounding error,
//   W[:, F] -= e_j / [H^-1]_jj [H^-1]_{j, F},   H = 2 X X^T,
// with one column order for all rows, lazily batched updates and the
// Cholesky form. With U the upper Cholesky factor of H^-1 (U^T U = H^-1) the
// step for column j is d = (w_j - w_hat_j) / U_jj, w_f -= d U_jf for f > j.
// Readings where the pages leave a step open: X is [t][k] (tokens x input
// channels); H is damped by 1 % of its mean diagonal (it is singular when
// t < k); U = V^-1 for the reverse Cholesky factor V of H (H = V V^T, V
// upper); weights are updated in fp32, each column's update applied to
// every later column as one fused multiply-add, in column order; a group's
// scale and zero come from its current (compensated) weights when its first
// column is reached, and codes round as the RTN quantizer does.
//
// Two entry points:
//  * the factor: X^T (bf16, zero-padded to 64 tokens) -> H = X^T X on bf16
//    MFMA -> 2 H + damping -> left-looking blocked reverse Cholesky in
//    64-wide panels (a panel's columns take the finished panels' terms in
//    one deep fp32 GEMM, its diagonal block is factored and inverted by one
//    wave, the panel above is solved by an fp32 GEMM) -> blocked inverse of
//    V -> U, all fp32;
//  * the column loop: per 128-column block, one wave per row walks the
//    block's columns with the block of U in LDS (the codes, the group's
//    scale and zero, the scaled errors d); then the later columns take the
//    block's updates as one fp32 GEMM, W[:, F] = W[:, F] - D U[block, F],
//    whose accumulator starts at W and adds the block's terms in column
//    order with fused multiply-adds -- the same operations, in the same
//    order, as applying each column's update as it is made.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

// --------------------------------------------------------------------------
// The column loop's update C[M][N] -= A[M][128] B[128][N] (A: the block's
// scaled errors, ld 128; B: the block's rows of U; C: the later columns of
// W). Each output starts at C and adds its 128 terms in ascending k with
// fused multiply-adds of -A (exact): the operations of applying each
// column's update as it is made.
// 128 x 128 tiles, 256 threads; thread (ty, tx) owns rows 4 ty + [0, 4) and
// 64 + 4 ty + [0, 4), columns 4 tx + [0, 4) and 64 + 4 tx + [0, 4), so its
// LDS reads are 16-byte and conflict-free. k in steps of 16 through two LDS
// buffers; the next step's loads are in registers during the current
// step's multiply-adds. N is a multiple of 128; rows past M are not stored.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void update128_kernel(int M, int N, const float *__restrict__ A,
                                                        const float *__restrict__ B, int64_t ldb,
                                                        float *__restrict__ C, int64_t ldc) {
    constexpr int T = 128, KS = 16;
    __shared__ __attribute__((aligned(16))) float As[2][KS][T];
    __shared__ __attribute__((aligned(16))) float Bs[2][KS][T];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
    // loads of one k step: A rows i0 + lr (two rows), k 4 lk .. + 3;
    // B row k0 + kb (two rows), columns j0 + 4 lc .. + 3
    const int lr = tid >> 2, lk = tid & 3;
    const int kb = tid >> 5, lc = tid & 31;
    f32x4 pa[2], pb[2];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // rows past M read row M - 1: they only feed outputs that are
            // not stored, and the loads need no branch
            const int i = min(i0 + lr + 64 * h, M - 1);
            pa[h] = *reinterpret_cast<const f32x4 *>(A + (int64_t)i * 128 + k0 + 4 * lk);
            pb[h] = *reinterpret_cast<const f32x4 *>(B + (int64_t)(k0 + kb + 8 * h) * ldb + j0 + 4 * lc);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = lr + 64 * h;
            As[buf][4 * lk + 0][row] = pa[h].x;
            As[buf][4 * lk + 1][row] = pa[h].y;
            As[buf][4 * lk + 2][row] = pa[h].z;
            As[buf][4 * lk + 3][row] = pa[h].w;
            *reinterpret_cast<f32x4 *>(&Bs[buf][kb + 8 * h][4 * lc]) = pb[h];
        }
    };
    float acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = min(i0 + 4 * ty + (r & 3) + 64 * (r >> 2), M - 1);  // rows past M: not stored
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 c4 = *reinterpret_cast<const f32x4 *>(C + (int64_t)i * ldc + j0 + 4 * tx + 64 * h);
            acc[r][4 * h + 0] = c4.x;
            acc[r][4 * h + 1] = c4.y;
            acc[r][4 * h + 2] = c4.z;
            acc[r][4 * h + 3] = c4.w;
        }
    }
    fetch(0);
    stash(0);
    __syncthreads();
    for (int step = 0; step < 128 / KS; ++step) {
        const int buf = step & 1;
        if (step + 1 < 128 / KS) fetch((step + 1) * KS);
        // (unrolled twice: a full unroll hoists every step's LDS reads into
        // registers and leaves one wave per SIMD)
#pragma unroll 2
        for (int kk = 0; kk < KS; ++kk) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&As[buf][kk][4 * ty]);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&As[buf][kk][64 + 4 * ty]);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&Bs[buf][kk][4 * tx]);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&Bs[buf][kk][64 + 4 * tx]);
            const float a[8] = {-a0.x, -a0.y, -a0.z, -a0.w, -a1.x, -a1.y, -a1.z, -a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
        }
        if (step + 1 < 128 / KS) stash(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = i0 + 4 * ty + (r & 3) + 64 * (r >> 2);
        if (i >= M) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<f32x4 *>(C + (int64_t)i * ldc + j0 + 4 * tx + 64 * h) =
                f32x4{acc[r][4 * h], acc[r][4 * h + 1], acc[r][4 * h + 2], acc[r][4 * h + 3]};
    }
}

// --------------------------------------------------------------------------
// fp32 GEMM on the matrix cores (v_mfma_f32_16x16x4f32) for the factor, where
// only fp32 accuracy matters (the column loop keeps the VALU update above,
// whose fixed accumulation order its codes depend on):
//   C[M][N] = (beta ? C : 0) + sgn * A[M][K] op(B),
// op(B) = B[K][N] (BT = false) or B^T with B given [N][K] (BT = true). M, N
// and K are multiples of 64 (the factor's panels). AUPPER:
// A is upper triangular, so row block i0 starts its sum at k = i0. PARTIAL:
// blockIdx.z takes the k range [z ksplit, (z + 1) ksplit) and writes its
// partial sum to C + z M N (ld N, no beta); sum_splits_kernel adds the
// partials in z order, so the result does not depend on scheduling.
// Block: 64 x 64 outputs, 4 waves of 32 x 32 (2 x 2 MFMA tiles); k in steps
// of 16 through LDS, the next step's loads in registers during the current
// step's MFMAs. MFMA operands: lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16] of a 16 x 16 x 4 step, and D rows 4 (l / 16) + v of
// column l % 16.
// --------------------------------------------------------------------------
template <bool BT, bool AUPPER, bool PARTIAL>
__global__ __launch_bounds__(256) void mgemm_kernel(int M, int N, int K, float sgn, const float *A, int64_t lda,
                                                    const float *B, int64_t ldb, int beta, float *C, int64_t ldc,
                                                    int ksplit) {
    // A tile [64 rows][16 k] at a row stride of 20 floats (16-byte aligned
    // rows, conflict-free fragment reads); B tile likewise when BT, else
    // [16 k][64 n] at a stride of 80 floats
    __shared__ __attribute__((aligned(16))) float As[64 * 20];
    __shared__ __attribute__((aligned(16))) float Bs[BT ? 64 * 20 : 16 * 80];
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, lq = lane >> 4;
    const int kb = max(AUPPER ? i0 : 0, PARTIAL ? (int)blockIdx.z * ksplit : 0);
    const int ke = PARTIAL ? min(K, ((int)blockIdx.z + 1) * ksplit) : K;
    if (PARTIAL) C += (int64_t)blockIdx.z * M * ldc;
    // this thread's 16-byte loads: A row tid / 4, k 4 (tid % 4); B the same
    // (BT) or k row tid / 16, n 4 (tid % 16)
    const int ar = tid >> 2, ak = 4 * (tid & 3);
    const int br = BT ? tid >> 2 : tid >> 4, bc = BT ? 4 * (tid & 3) : 4 * (tid & 15);
    const float *ap = A + (int64_t)(i0 + ar) * lda + ak;
    const float *bp = BT ? B + (int64_t)(j0 + br) * ldb + bc : B + (int64_t)br * ldb + j0 + bc;
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[mt][nt][v] = beta && !PARTIAL
                                     ? C[(int64_t)(i0 + wm * 32 + mt * 16 + 4 * lq + v) * ldc + j0 + wn * 32 + nt * 16 + l16]
                                     : 0.0f;
    // an empty k range (a split wholly below a triangular A's row block)
    // still writes its zero partial
    f32x4 ra = f32x4{0.f, 0.f, 0.f, 0.f}, rb = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb < ke) {
        ra = *reinterpret_cast<const f32x4 *>(ap + kb);
        rb = BT ? *reinterpret_cast<const f32x4 *>(bp + kb) : *reinterpret_cast<const f32x4 *>(bp + (int64_t)kb * ldb);
    }
    for (int k0 = kb; k0 < ke; k0 += 16) {
        *reinterpret_cast<f32x4 *>(&As[ar * 20 + ak]) = ra;
        if (BT)
            *reinterpret_cast<f32x4 *>(&Bs[br * 20 + bc]) = rb;
        else
            *reinterpret_cast<f32x4 *>(&Bs[br * 80 + bc]) = rb;
        __syncthreads();
        if (k0 + 16 < ke) {
            ra = *reinterpret_cast<const f32x4 *>(ap + k0 + 16);
            rb = BT ? *reinterpret_cast<const f32x4 *>(bp + k0 + 16)
                    : *reinterpret_cast<const f32x4 *>(bp + (int64_t)(k0 + 16) * ldb);
        }
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
            float a[2], b[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) a[mt] = sgn * As[(wm * 32 + mt * 16 + l16) * 20 + kk + lq];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                b[nt] = BT ? Bs[(wn * 32 + nt * 16 + l16) * 20 + kk + lq] : Bs[(kk + lq) * 80 + wn * 32 + nt * 16 + l16];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                C[(int64_t)(i0 + wm * 32 + mt * 16 + 4 * lq + v) * ldc + j0 + wn * 32 + nt * 16 + l16] = acc[mt][nt][v];
}

template <bool BT, bool AUPPER>
hipError_t mgemm(int64_t M, int64_t N, int64_t K, float sgn, const float *A, int64_t lda, const float *B, int64_t ldb,
                 int beta, float *C, int64_t ldc, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (M % 64 || N % 64 || K % 64) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)(N / 64), (uint32_t)(M / 64));
    hipLaunchKernelGGL((mgemm_kernel<BT, AUPPER, false>), grid, dim3(256), 0, st, (int)M, (int)N, (int)K, sgn,
                       A, lda, B, ldb, beta, C, ldc, 0);
    return hipGetLastError();
}

constexpr int kMaxSplits = 16;  // k ranges of the narrow, deep products

// C[i][j] = (beta ? C[i][j] : 0) + sum over z of part[z][i][j], z in order.
// Every partial is loaded before the first addition (a loop over a runtime
// count waited for each load in turn).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float *__restrict__ part, int splits, int M, int N,
                                                         int beta, float *__restrict__ C, int64_t ldc) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)M * N) return;
    const int i = (int)(e / N), j = (int)(e % N);
    float pv[kMaxSplits];
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z) pv[z] = part[(int64_t)min(z, splits - 1) * M * N + e];  // past splits: unused
    float v = beta ? C[(int64_t)i * ldc + j] : 0.0f;
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z)
        if (z < splits) v += pv[z];
    C[(int64_t)i * ldc + j] = v;
}

// A narrow product (N = 64) with a deep k: k split into up to kMaxSplits
// ranges of at least 128, as many as bring the launch to about 2048
// workgroups (measured: ranges of at least 1024 left the factor's first
// panels a few long-running workgroups); the partials go to part
// (kMaxSplits M N floats) and are added, in order, to beta ? C : 0.
template <bool BT, bool AUPPER>
hipError_t mgemm_deep(int64_t M, int64_t N, int64_t K, float sgn, const float *A, int64_t lda, const float *B,
                      int64_t ldb, int beta, float *C, int64_t ldc, float *part, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (M % 64 || N % 64 || K % 64) return hipErrorInvalidValue;
    const int64_t tiles = (M / 64) * (N / 64);
    const int splits = (int)std::min<int64_t>(
        std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, K / 128)), std::max<int64_t>(1, 2048 / tiles));
    if (splits == 1) return mgemm<BT, AUPPER>(M, N, K, sgn, A, lda, B, ldb, beta, C, ldc, st);
    const int64_t ksplit = (K / 64 + splits - 1) / splits * 64;
    const dim3 grid((uint32_t)(N / 64), (uint32_t)(M / 64), (uint32_t)splits);
    hipLaunchKernelGGL((mgemm_kernel<BT, AUPPER, true>), grid, dim3(256), 0, st, (int)M, (int)N, (int)K, sgn, A,
                       lda, B, ldb, 0, part, N, (int)ksplit);
    hipLaunchKernelGGL(sum_splits_kernel, dim3((uint32_t)((M * N + 255) / 256)), dim3(256), 0, st, part, splits, (int)M,
                       (int)N, beta, C, ldc);
    return hipGetLastError();
}

// X [t][k] bf16 -> X^T [k][tp] bf16, tokens t .. tp - 1 zero (tp a multiple of 64).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ x, int t, int k, int tp,
                                                             uint16_t *__restrict__ xt) {
    __shared__ uint16_t tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;  // c: channel, r: token
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int yy = ty; yy < 32; yy += 8) {
        const int r = r0 + yy, c = c0 + tx;
        tile[yy][tx] = r < t && c < k ? x[(int64_t)r * k + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int yy = ty; yy < 32; yy += 8) {
        const int c = c0 + yy, r = r0 + tx;
        if (c < k && r < tp) xt[(int64_t)c * tp + r] = tile[tx][yy];
    }
}

// H = 2 H, then H_ii += percdamp * mean(H_ii): the diagonal's sum in fp64 by
// one workgroup, in a fixed order.
__global__ __launch_bounds__(256) void damp_sum_kernel(const float *__restrict__ h, int k, double *__restrict__ sum) {
    __shared__ double lds[256];
    double acc = 0.0;
    for (int i = threadIdx.x; i < k; i += 256) acc += 2.0 * (double)h[(int64_t)i * k + i];
    lds[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) lds[threadIdx.x] += lds[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *sum = lds[0];
}

__global__ __launch_bounds__(256) void damp_apply_kernel(float *__restrict__ h, int k, float percdamp,
                                                         const double *__restrict__ sum) {
    const int64_t total = (int64_t)k * k;
    const float lam = (float)((double)percdamp * (*sum / (double)k));
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / k, j = e % k;
        h[e] = 2.0f * h[e] + (i == j ? lam : 0.0f);
    }
}

constexpr int NB = 64;  // panel width of the factorisation

// The diagonal block B = [j0, j0 + 64) of the (updated) H: reverse Cholesky
// V_BB (H_BB = V_BB V_BB^T, upper) written back into H's block, and its
// inverse into vinv (64 x 64, zeros below the diagonal). One wave, no
// barriers: LDS operations of a wave complete in order, so a column written
// to LDS is read back by every lane in the same step.
//  * Cholesky, column j from the last: lane i holds row i of the working
//    block A in registers. F_ij = A_ij / sqrt(A_jj) (F_jj = sqrt(A_jj), the
//    same product A_jj rsqrt(A_jj)), then A_il -= F_ij F_lj for l < j, with
//    column j of F broadcast through LDS (two columns per broadcast); lane
//    i's register j then holds F_ij.
//  * inverse W = F^-1 from W = I, row m from the last: lane c holds column c
//    of W; W_mc /= F_mm, then W_ic -= F_im W_mc for i < m, reading column m
//    of F from a column-major copy of F written to LDS once.
// Both loops unroll fully, so every register index is a constant. Rows and
// columns of a lane outside the triangle it owns are updated too: they are
// never read as results. Measured on MI355X: 54 us per block with four
// waves and a barrier per step.
__global__ __launch_bounds__(64) void chol_diag_kernel(float *__restrict__ h, int k, int j0,
                                                       float *__restrict__ vinv) {
    __shared__ __attribute__((aligned(16))) float col[NB];
    __shared__ __attribute__((aligned(16))) float col2[NB];
    __shared__ __attribute__((aligned(16))) float Fc[NB][NB];
    const int lane = threadIdx.x;
    // always 1, but opaque to the compiler: each unrolled step below sits in
    // its own (never skipped) branch, which keeps the straight-line blocks
    // short enough for the code generator (one 7000-instruction block took
    // it minutes to compile)
    int go;
    asm volatile("s_mov_b32 %0, 1" : "=s"(go));
    float a[NB];
    // row `lane` of the symmetric block, from its current upper triangle
#pragma unroll
    for (int l = 0; l < NB; ++l)
        a[l] = lane <= l ? h[(int64_t)(j0 + lane) * k + j0 + l] : h[(int64_t)(j0 + l) * k + j0 + lane];
#pragma unroll
    // columns in pairs (j, j - 1), j odd: column j's term on column j - 1
    // goes through readlane, then both columns are broadcast through LDS
    // together (one write-to-read round trip per pair); every element takes
    // column j's term, then column j - 1's, as one column at a time would
    for (int jj = NB / 2 - 1; jj >= 0; --jj) {
        if (!go) continue;
        const int j = 2 * jj + 1;
        // hardware 1 / sqrt (about 1 ulp; the factor needs fp32 accuracy,
        // not correct rounding); not positive definite: NaN or inf, which
        // propagates to U
        const float ajj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j]), j));
        const float f = a[j] * __builtin_amdgcn_rsqf(ajj);
        a[j] = f;
        const float fj1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j - 1));  // F_{j-1, j}
        a[j - 1] = __builtin_fmaf(-f, fj1, a[j - 1]);
        const float aj1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j - 1]), j - 1));
        const float g = a[j - 1] * __builtin_amdgcn_rsqf(aj1);
        a[j - 1] = g;
        col[lane] = f;
        col2[lane] = g;
#pragma unroll
        for (int l = (j - 2) & ~3; l >= 0; l -= 4) {
            const f32x4 c4 = *reinterpret_cast<const f32x4 *>(&col[l]);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&col2[l]);
            if (l + 3 < j - 1) a[l + 3] = __builtin_fmaf(-g, d4.w, __builtin_fmaf(-f, c4.w, a[l + 3]));
            if (l + 2 < j - 1) a[l + 2] = __builtin_fmaf(-g, d4.z, __builtin_fmaf(-f, c4.z, a[l + 2]));
            if (l + 1 < j - 1) a[l + 1] = __builtin_fmaf(-g, d4.y, __builtin_fmaf(-f, c4.y, a[l + 1]));
            a[l] = __builtin_fmaf(-g, d4.x, __builtin_fmaf(-f, c4.x, a[l]));
        }
    }
    // V_BB = F back into H's block (upper triangle: row lane, columns >= lane)
#pragma unroll
    for (int l = 0; l < NB; ++l)
        if (lane <= l) h[(int64_t)(j0 + lane) * k + j0 + l] = a[l];
    // F column-major in LDS (Fc[l][i] = F_il), written once: the inverse's
    // steps then only read
#pragma unroll
    for (int l = 0; l < NB; ++l) Fc[l][lane] = a[l];
    float w[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) w[i] = i == lane ? 1.0f : 0.0f;
#pragma unroll
    for (int m = NB - 1; m >= 0; --m) {
        if (!go) continue;
        const float fmm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[m]), m));
        w[m] *= __builtin_amdgcn_rcpf(fmm);
#pragma unroll
        for (int i = (m - 1) & ~3; i >= 0; i -= 4) {
            const f32x4 c4 = *reinterpret_cast<const f32x4 *>(&Fc[m][i]);
            if (i + 3 < m) w[i + 3] = __builtin_fmaf(-c4.w, w[m], w[i + 3]);
            if (i + 2 < m) w[i + 2] = __builtin_fmaf(-c4.z, w[m], w[i + 2]);
            if (i + 1 < m) w[i + 1] = __builtin_fmaf(-c4.y, w[m], w[i + 1]);
            w[i] = __builtin_fmaf(-c4.x, w[m], w[i]);
        }
    }
#pragma unroll
    for (int m = 0; m < NB; ++m) vinv[m * NB + lane] = lane >= m ? w[m] : 0.0f;
}

__global__ __launch_bounds__(256) void fill_kernel(float *__restrict__ p, int64_t count) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) p[e] = 0.0f;
}

// U[j0:j0+64][j0:j0+64] = vinv block
__global__ __launch_bounds__(256) void put_block_kernel(const float *__restrict__ blk, float *__restrict__ u, int k,
                                                        int j0) {
    for (int e = threadIdx.x; e < NB * NB; e += 256) u[(int64_t)(j0 + e / NB) * k + j0 + e % NB] = blk[e];
}

__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const uint16_t *__restrict__ w, int64_t count,
                                                          float *__restrict__ out) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256)
        out[e] = bf16_lo((uint32_t)w[e]);
}

// --------------------------------------------------------------------------
// The column loop of one 128-column block. One wave per row, lane l holding
// columns j0 + l and j0 + 64 + l of the compensated row; the block of U
// (128 x 128) in LDS, shared by the workgroup's 16 rows.
// --------------------------------------------------------------------------
constexpr int GB = 128;  // columns per block (the lazy batch)

// The definition's clamp on a finite value (inputs are finite): v_med3, one
// instruction in the serial per-column chain instead of two compares and two
// selects.
LQ_DEVICE float clampf_def(float v, float lo, float hi) { return __builtin_amdgcn_fmed3f(v, lo, hi); }

template <int BITS, bool SYM>
__global__ __launch_bounds__(1024) void gptq_block_kernel(float *__restrict__ w, int n, int k,
                                                          const float *__restrict__ u, int j0, int group,
                                                          float *__restrict__ dbuf, uint8_t *__restrict__ codes,
                                                          float *__restrict__ scales, float *__restrict__ zeros) {
    __shared__ float Us[GB][GB + 1];
    for (int e = threadIdx.x; e < GB * GB; e += 1024)
        Us[e / GB][e % GB] = u[(int64_t)(j0 + e / GB) * k + j0 + e % GB];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 16 + (threadIdx.x >> 6);
    if (r >= n) return;  // no barrier follows
    float *row = w + (int64_t)r * k;
    float a = row[j0 + lane], b = row[j0 + 64 + lane];
    const int ng = k / group;
    const int g = j0 / group;
    float s, z;
    if (j0 % group == 0) {
        // the group's scale and zero from its current weights (the RTN formulas)
        float mn = fminf(a, b), mx = fmaxf(a, b), am = fmaxf(fabsf(a), fabsf(b));
        for (int c = j0 + 128 + lane; c < j0 + group; c += 64) {
            const float v = row[c];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
            am = fmaxf(am, fabsf(v));
        }
        if (SYM) {
            am = team_max<64>(am);
            if (am < kFloor) am = kFloor;
            s = am / (float)((1 << (BITS - 1)) - 1);
            z = 0.0f;
        } else {
            mn = team_min<64>(mn);
            mx = team_max<64>(mx);
            float range = mx - mn;
            if (range < kFloor) range = kFloor;
            s = range / (float)((1 << BITS) - 1);
            z = rintf(-mn / s) + 0.0f;
        }
        if (lane == 0) {
            scales[(int64_t)r * ng + g] = s;
            if (!SYM) zeros[(int64_t)r * ng + g] = z;
        }
    } else {
        s = scales[(int64_t)r * ng + g];
        z = SYM ? 0.0f : zeros[(int64_t)r * ng + g];
    }
    int qa = 0, qb = 0;
    float da = 0.0f, db = 0.0f;
    // Column j: its code and scaled error d from the current value, then every
    // lane's columns take fma(-d, U_jf, w_f). U is zero below its diagonal,
    // so that update leaves the columns before j unchanged, and column j's own
    // value is not read again once its code and d are taken: no lane needs a
    // predicate. Columns 0..63 sit in a, 64..127 in b.
    auto step = [&](int j, float wj, float &q_keep, float &d_keep) {
        float qf;
        if (SYM) {
            const float top = (float)((1 << (BITS - 1)) - 1);
            qf = clampf_def(rintf(wj / s), -top, top);
        } else {
            const float top = (float)((1 << BITS) - 1);
            qf = clampf_def(rintf(wj / s) + z, 0.0f, top);
        }
        const float d = (wj - (qf - z) * s) / Us[j][j];
        a = __builtin_fmaf(-d, Us[j][lane], a);
        b = __builtin_fmaf(-d, Us[j][64 + lane], b);
        if (lane == (j & 63)) {
            q_keep = qf;
            d_keep = d;
        }
    };
    float qfa = 0.0f, qfb = 0.0f;
    for (int j = 0; j < 64; ++j) step(j, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), j)), qfa, da);
    for (int j = 64; j < GB; ++j) step(j, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), j - 64)), qfb, db);
    qa = (int)qfa;
    qb = (int)qfb;
    dbuf[(int64_t)r * GB + lane] = da;
    dbuf[(int64_t)r * GB + 64 + lane] = db;
    if (BITS == 4) {
        const int ua = SYM ? qa + 8 : qa, ub = SYM ? qb + 8 : qb;
        // element 2i in the low nibble: lane 2i takes its odd neighbour's code
        const int na = __shfl_xor(ua, 1), nb = __shfl_xor(ub, 1);
        if ((lane & 1) == 0) {
            uint8_t *cr = codes + (int64_t)r * (k / 2);
            cr[(j0 + lane) / 2] = (uint8_t)((ua & 0xF) | ((na & 0xF) << 4));
            cr[(j0 + 64 + lane) / 2] = (uint8_t)((ub & 0xF) | ((nb & 0xF) << 4));
        }
    } else {
        uint8_t *cr = codes + (int64_t)r * k;
        cr[j0 + lane] = (uint8_t)qa;
        cr[j0 + 64 + lane] = (uint8_t)qb;
    }
}

constexpr int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

int64_t gptq_factor_workspace_bytes(int64_t t, int64_t k) {
    const int64_t tp = (t + 63) / 64 * 64;
    return align256(k * tp * 2) + align256(k * k * 4) + align256(k * NB * 4) + align256(k * NB * 4) + 256 +
           align256(kMaxSplits * k * NB * 4);
}

int64_t gptq_quantize_workspace_bytes(int64_t n, int64_t k) { return align256(n * k * 4) + align256(n * GB * 4); }

hipError_t launch_gptq_factor(const uint16_t *x, int64_t t, int64_t k, float percdamp, void *workspace, float *u,
                              hipStream_t st) {
    const int64_t tp = (t + 63) / 64 * 64;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *xt = reinterpret_cast<uint16_t *>(ws);
    ws += align256(k * tp * 2);
    float *h = reinterpret_cast<float *>(ws);
    ws += align256(k * k * 4);
    float *vinv = reinterpret_cast<float *>(ws);  // [k / 64][64][64]
    ws += align256(k * NB * 4);
    float *tmp = reinterpret_cast<float *>(ws);  // [k][64]
    ws += align256(k * NB * 4);
    double *dsum = reinterpret_cast<double *>(ws);
    ws += 256;
    float *part = reinterpret_cast<float *>(ws);  // [kMaxSplits][k][64]
    hipError_t e;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((uint32_t)((k + 31) / 32), (uint32_t)(tp / 32)), dim3(256), 0, st,
                       x, (int)t, (int)k, (int)tp, xt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_gemm_bf16(xt, xt, k, k, tp, h, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(damp_sum_kernel, dim3(1), dim3(256), 0, st, h, (int)k, dsum);
    hipLaunchKernelGGL(damp_apply_kernel, dim3(2048), dim3(256), 0, st, h, (int)k, percdamp, dsum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int panels = (int)(k / NB);
    // reverse Cholesky, last panel first, left-looking: the panel's columns
    // take all finished panels' contributions in one deep product,
    //   H[0 : j0 + 64, B] -= V[0 : j0 + 64, D] V[B, D]^T   (D: columns >= j0 + 64),
    // then its diagonal block is factored and V_AB = H_AB Vinv_BB^T. (Applying
    // each panel's rank-64 update to the whole remaining triangle instead
    // reads and writes that triangle once per panel: twice the memory traffic,
    // 31 % of the factor's time at k = 11008.) V's columns stay in H's upper
    // triangle; the lower triangles of diagonal blocks are never read.
    for (int p = panels - 1; p >= 0; --p) {
        const int64_t j0 = (int64_t)p * NB;
        const int64_t kd = k - j0 - NB;
        if (kd > 0 && (e = mgemm_deep<true, false>(j0 + NB, NB, kd, -1.0f, h + j0 + NB, k, h + j0 * k + j0 + NB, k, 1,
                                                    h + j0, k, part, st)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(64), 0, st, h, (int)k, (int)j0, vinv + p * NB * NB);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (j0 == 0) continue;
        // V_AB = H_AB Vinv_BB^T (in place: each workgroup owns 64 rows and
        // reads all of them before it writes)
        if ((e = mgemm<true, false>(j0, NB, NB, 1.0f, h + j0, k, vinv + p * NB * NB, NB, 0, h + j0, k, st)) !=
            hipSuccess)
            return e;
    }
    // U = V^-1, first panel first: U_BB = Vinv_BB, U_AB = -U_AA (V_AB U_BB)
    hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(256), 0, st, u, k * k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int p = 0; p < panels; ++p) {
        const int64_t j0 = (int64_t)p * NB;
        hipLaunchKernelGGL(put_block_kernel, dim3(1), dim3(256), 0, st, vinv + p * NB * NB, u, (int)k, (int)j0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (j0 == 0) continue;
        if ((e = mgemm<false, false>(j0, NB, NB, 1.0f, h + j0, k, u + j0 * k + j0, k, 0, tmp, NB, st)) !=
            hipSuccess)
            return e;
        // U_AA is upper triangular: row block i0 sums from k = i0
        if ((e = mgemm_deep<false, true>(j0, NB, j0, -1.0f, u, k, tmp, NB, 0, u + j0, k, part, st)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free column loop (gptq_quantize_noalloc): a
// file-scope device array. Every device the library runs on holds its own
// copy of it until the process ends. In host code the name `scratch` is only
// a host-side stand-in for the symbol, so host code never passes it to a
// kernel; it uses the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
constexpr int64_t kStaticScratchBytes = int64_t(72) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
}  // namespace

int64_t gptq_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t gptq_static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_gptq_quantize(const GptqArgs &a, hipStream_t st) {
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    float *wf = reinterpret_cast<float *>(ws);
    ws += align256(a.n * a.k * 4);
    float *dbuf = reinterpret_cast<float *>(ws);
    hipError_t e;
    hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(4096), dim3(256), 0, st, a.w, a.n * a.k, wf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint32_t blocks = (uint32_t)((a.n + 15) / 16);
    for (int64_t j0 = 0; j0 < a.k; j0 += GB) {
#define LQ_GPTQ_BLOCK(BITS, S)                                                                                     \
    hipLaunchKernelGGL((gptq_block_kernel<BITS, S>), dim3(blocks), dim3(1024), 0, st, wf, (int)a.n, (int)a.k, a.u, \
                       (int)j0, (int)a.group, dbuf, a.codes, a.scales, a.zeros)
        if (a.bits == 4 && a.symmetric) LQ_GPTQ_BLOCK(4, true);
        else if (a.bits == 4) LQ_GPTQ_BLOCK(4, false);
        else if (a.symmetric) LQ_GPTQ_BLOCK(8, true);
        else LQ_GPTQ_BLOCK(8, false);
#undef LQ_GPTQ_BLOCK
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t f0 = j0 + GB;
        if (f0 < a.k) {
            // W[:, f0:] = W[:, f0:] - D U[j0:j0+128, f0:], in column order per element
            const dim3 grid((uint32_t)((a.k - f0) / 128), (uint32_t)((a.n + 127) / 128));
            hipLaunchKernelGGL(update128_kernel, grid, dim3(256), 0, st, (int)a.n, (int)(a.k - f0), dbuf,
                               a.u + j0 * a.k + f0, a.k, wf + f0, a.k);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace lq
