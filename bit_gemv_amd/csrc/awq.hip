// awq.hip -- AWQ activation-aware scale search on gfx950.
//
// Method ("3.6 Quantization", AWQ section: protect the weight channels that
// multiply large activations by scaling them before RTN,
//   y = sum_j (s_j w_j)(x_j / s_j) -> sum_j quant(s_j w_j) x_j / s_j,
// with s = s_X^alpha, s_X the mean activation magnitude of each input channel
// over calibration data, and alpha grid-searched over [0, 1] per layer to
// minimise the layer's output error; 1/s is folded into the preceding op.
// PTQ concept page, AWQ steps 1-5: calibrate |X| per channel, W' = W diag(s),
// plain RTN of W', inference Y = X diag(s)^-1 quant(W')).
// Readings where the pages leave a step open: alpha_i = i / n_grid for
// i = 0..n_grid; s_X floored at 1e-8 before the power; the activations reach
// the quantized product as bf16(x / s); the output error is the squared
// Frobenius norm of X W^T - X' W_hat'^T over the calibration tokens; ties
// keep the smallest alpha.
//
// The search is a loop of data-parallel passes, all on the device and on one
// stream (no host synchronisation):
//   once:      Y = X W^T                     (gemm_bf16_kernel, bf16 MFMA)
//   per alpha: s = powf(max(s_X, 1e-8), alpha)        (awq_scale_kernel)
//              X' = bf16(X / s)                        (div_act_kernel)
//              quant(W diag(s))                        (the group-wise quantizer)
//              Y' = X' W_hat'^T                        (the W4A16 GEMM)
//              loss = sum (Y - Y')^2                   (in the GEMM's epilogue, fp64)
//   then:      argmin, s_best, quant(W diag(s_best))   (awq_pick_kernel + quantizer)
// Channel magnitudes s_X come from act_absmean_kernel (a separate entry
// point, so the caller can reuse them across the layer's linears).
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// --------------------------------------------------------------------------
// s_X[j] = (sum_t |X[t][j]|) / t, the sum in fp64. Block: 64 columns x 4
// row strides; the fp64 partials of the four waves are added in a fixed
// order, so the result does not depend on the launch. (The sum of bf16
// magnitudes is exact in fp64 unless the values span more than ~2^44, so in
// practice it equals the sum in any order.)
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void act_absmean_kernel(const uint16_t *__restrict__ x, int t, int k,
                                                          float *__restrict__ sx) {
    __shared__ double part[4][64];
    const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + c;
    double acc = 0.0;
    if (col < k)
        for (int r = r0; r < t; r += 4) acc += (double)fabsf(bf16_lo((uint32_t)x[(int64_t)r * k + col]));
    part[r0][c] = acc;
    __syncthreads();
    if (r0 == 0 && col < k) {
        const double s = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
        sx[col] = (float)(s / (double)t);
    }
}

// The candidate scale of grid point i (shared by the search and the pick, so
// both produce the same bits).
LQ_DEVICE float awq_scale_of(float sxj, int i, int n_grid) {
    const float alpha = (float)i / (float)n_grid;
    return powf(sxj < kFloor ? kFloor : sxj, alpha);
}

// Grid point i0 + blockIdx.y; its scales at s + blockIdx.y * s_stride.
__global__ __launch_bounds__(256) void awq_scale_kernel(const float *__restrict__ sx, int k, int i0, int n_grid,
                                                        float *__restrict__ s, int64_t s_stride) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j < k) s[blockIdx.y * s_stride + j] = awq_scale_of(sx[j], i0 + (int)blockIdx.y, n_grid);
}

// fp32 -> bf16 bits, round to nearest even (finite values).
LQ_DEVICE uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// X'[t][j] = bf16(X[t][j] / s[j]) (IEEE division). One thread per 8
// consecutive activations (one 16-byte load and store); k is a multiple of 8.
// Grid point blockIdx.y: s and X' at blockIdx.y times their strides.
__global__ __launch_bounds__(256) void div_act_kernel(const uint16_t *__restrict__ x, int64_t total8, int k,
                                                      const float *__restrict__ s, int64_t s_stride,
                                                      uint16_t *__restrict__ xa, int64_t x_stride) {
    s += blockIdx.y * s_stride;
    xa += blockIdx.y * x_stride;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total8; i += (int64_t)gridDim.x * 256) {
        const u32x4 v = reinterpret_cast<const u32x4 *>(x)[i];
        const int j0 = (int)((i * 8) % k);
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(s + j0);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(s + j0 + 4);
        u32x4 o;
        o.x = bf16_rne(bf16_lo(v.x) / s0.x) | (bf16_rne(bf16_hi(v.x) / s0.y) << 16);
        o.y = bf16_rne(bf16_lo(v.y) / s0.z) | (bf16_rne(bf16_hi(v.y) / s0.w) << 16);
        o.z = bf16_rne(bf16_lo(v.z) / s1.x) | (bf16_rne(bf16_hi(v.z) / s1.y) << 16);
        o.w = bf16_rne(bf16_lo(v.w) / s1.z) | (bf16_rne(bf16_hi(v.w) / s1.w) << 16);
        reinterpret_cast<u32x4 *>(xa)[i] = o;
    }
}

// --------------------------------------------------------------------------
// Squared error sum((Y - Y')^2) in fp64: per-block partials over a fixed
// grid-stride assignment, then one block adds them in a fixed order.
// --------------------------------------------------------------------------
LQ_DEVICE double block_sum(double v, double *lds) {
    // 256 threads: tree through LDS in a fixed order
    lds[threadIdx.x] = v;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) lds[threadIdx.x] += lds[threadIdx.x + w];
        __syncthreads();
    }
    return lds[0];
}

// Argmin over the grid (first minimum), then s_best and the index.
__global__ __launch_bounds__(256) void awq_pick_kernel(const double *__restrict__ losses, int n_grid,
                                                       const float *__restrict__ sx, int k,
                                                       float *__restrict__ s_best, int32_t *__restrict__ best) {
    int arg = 0;
    for (int i = 1; i <= n_grid; ++i)
        if (losses[i] < losses[arg]) arg = i;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j < k) s_best[j] = awq_scale_of(sx[j], arg, n_grid);
    if (blockIdx.x == 0 && threadIdx.x == 0) *best = arg;
}

// --------------------------------------------------------------------------
// Y[m][n] = X[m][k] W[n][k]^T, bf16 inputs, fp32 output (the unquantized
// layer output the search compares against). v_mfma_f32_16x16x32_bf16, a
// block of 4 waves computes 128 x 128 outputs (2 x 2 waves of 64 x 64) and
// walks k 64 at a time. A stage's X and W tiles (16 KB each) go from memory
// straight into a 3-slot LDS ring with buffer loads in the LDS-write form,
// two stages ahead. LDS rows are 128 bytes; 16-byte chunk c of row r is
// stored at c ^ ((r >> 1) & 7), so the 16 rows a fragment read touches fall
// in distinct banks. MFMA k-step j (0, 1) gives lane quarter kq the
// activations and weights k = 16 kq + 8 j + [0, 8) of the stage: A and B
// use the same order, so the contraction is unchanged.
// --------------------------------------------------------------------------
constexpr int GB_M = 128, GB_N = 128, GB_K = 64, GB_STAGES = 3;
constexpr int GB_TILE = GB_M * GB_K * 2;  // one operand tile of a stage
constexpr int GB_SLOT = 2 * GB_TILE;
// vmcnt literal of the stage wait: one younger stage of 8 loads per wave
#define LQ_GB_VM_STEP 8
static_assert(LQ_GB_VM_STEP == (GB_STAGES - 2) * (GB_SLOT / 1024 / 4), "stage wait vmcnt");
#define LQ_GB_STR2(x) #x
#define LQ_GB_STR(x) LQ_GB_STR2(x)

LQ_DEVICE int gb_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                        int m, int n, int k, float *__restrict__ y) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[GB_STAGES][GB_SLOT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, kq = lane >> 4;

    // XCD-aware order: the blocks that share a 128-row slice of W run on one XCD
    const int nt_count = (n + GB_N - 1) / GB_N, mt_count = (m + GB_M - 1) / GB_M;
    int tn, tm;
    if ((nt_count & 7) == 0) {
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        tn = xcd * (nt_count >> 3) + idx / mt_count;
        tm = idx % mt_count;
    } else {
        tn = blockIdx.x % nt_count;
        tm = blockIdx.x / nt_count;
    }
    const int n0 = tn * GB_N, m0 = tm * GB_M;
    const int nst = k / GB_K;
    const int rows_m = min(GB_M, m - m0), rows_n = min(GB_N, n - n0);
    // rows past m or n read zeros; their outputs are never stored
    const auto rx = make_rsrc(x + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k * 2);
    const auto rw = make_rsrc(w + (int64_t)n0 * k, (uint32_t)rows_n * (uint32_t)k * 2);

    // this wave's 8 pieces of 1 KB (8 rows x 128 B) per stage: waves 0, 1 the
    // X tile, waves 2, 3 the W tile; lane l: row 8 p + l / 8 of the tile,
    // physical chunk l % 8 holding logical chunk (l % 8) ^ swz(row)
    uint32_t src_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = 8 * (wave & 1) + i;
        const int row = 8 * p + (lane >> 3);
        src_off[i] = (uint32_t)row * (uint32_t)k * 2 + 16u * (uint32_t)((lane & 7) ^ gb_swz(row));
    }
    auto issue = [&](int st) {
        uint8_t *slot = ring[st % GB_STAGES] + (wave < 2 ? 0 : GB_TILE);
        const bool in = st < nst;  // later stages only keep the load count uniform
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wave < 2 ? rx : rw, (__attribute__((address_space(3))) void *)(slot + 1024 * (8 * (wave & 1) + i)),
                16, in ? src_off[i] + (uint32_t)st * (GB_K * 2) : kOutOfRange, 0, 0, 0);
    };

    int a_off[4][2], b_off[4][2];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ra = wm * 64 + t4 * 16 + l16, rb = wn * 64 + t4 * 16 + l16;
            a_off[t4][j] = ra * (GB_K * 2) + 16 * ((2 * kq + j) ^ gb_swz(ra));
            b_off[t4][j] = GB_TILE + rb * (GB_K * 2) + 16 * ((2 * kq + j) ^ gb_swz(rb));
        }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < GB_STAGES - 1; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
        // this wave's loads of stage st are done once one younger stage's are
        // pending; after the barrier every wave's are, and every wave has
        // finished stage st - 1, whose slot the issue below refills
        asm volatile("s_waitcnt vmcnt(" LQ_GB_STR(LQ_GB_VM_STEP) ")\n\ts_barrier" ::: "memory");
        issue(st + GB_STAGES - 1);
        const uint8_t *slot = ring[st % GB_STAGES];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bf16x8_t a[4], b[4];
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                a[t4] = *reinterpret_cast<const bf16x8_t *>(slot + a_off[t4][j]);
                b[t4] = *reinterpret_cast<const bf16x8_t *>(slot + b_off[t4][j]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    }
    // drain the trailing (out-of-range) loads; tells the compiler nothing is pending
    __builtin_amdgcn_s_waitcnt(0x0F70);
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

constexpr int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t m, int64_t n, int64_t k, float *y,
                            hipStream_t st) {
    const uint32_t blocks = (uint32_t)(((n + GB_N - 1) / GB_N) * ((m + GB_M - 1) / GB_M));
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(blocks), dim3(256), 0, st, a, b, (int)m, (int)n, (int)k, y);
    return hipGetLastError();
}

// Grid points evaluated per batch: their quantized weights and scaled
// activations sit side by side in the workspace, and one launch of the
// W4A16 GEMM computes all their products with the squared error against
// the reference product fused into its epilogue (at n = 4096 one product
// alone is only 128 workgroups). Measured on MI355X, 512 tokens, 21 grid
// points, per linear: batches of 11 took 1.30 / 3.01 / 2.94 ms on
// 4096 x 4096 / 11008 x 4096 / 4096 x 11008, batches of 4 1.39 / 3.45 /
// 3.18 ms, one batch of 21 1.31 / 3.20 / 3.13 ms.
constexpr int kAwqBatch = 11;

int64_t awq_workspace_bytes(int64_t t, int64_t n, int64_t k) {
    const int64_t meta = n * (k / 128) * 4;  // scales (or zeros) of one point, group >= 128
    return align256(t * n * 4) + kAwqBatch * (align256(t * k * 2) + align256(k * 4) + align256(n * k / 2) +
                                              2 * align256(meta)) +
           align256(kAwqBatch * w4a16_gemm_blocks(t, n) * 8);
}

hipError_t launch_act_absmean(const uint16_t *x, int64_t t, int64_t k, float *sx, hipStream_t st) {
    hipLaunchKernelGGL(act_absmean_kernel, dim3((uint32_t)((k + 63) / 64)), dim3(256), 0, st, x, (int)t, (int)k, sx);
    return hipGetLastError();
}

// The loss of grid point z: the workgroup partials of its product, summed
// in a fixed order.
__global__ __launch_bounds__(256) void loss_finish_kernel(const double *__restrict__ partials, int64_t blocks,
                                                          double *__restrict__ out) {
    __shared__ double lds[256];
    const double *p = partials + (int64_t)blockIdx.x * blocks;
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < blocks; i += 256) acc += p[i];
    const double s = block_sum(acc, lds);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

hipError_t launch_awq_search(const AwqArgs &a, hipStream_t st) {
    const int64_t meta = a.n * (a.k / 128) * 4;
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    float *y_ref = reinterpret_cast<float *>(ws);
    ws += align256(a.t * a.n * 4);
    uint16_t *xa = reinterpret_cast<uint16_t *>(ws);  // [kAwqBatch][t][k]
    ws += kAwqBatch * align256(a.t * a.k * 2);
    float *s = reinterpret_cast<float *>(ws);  // [kAwqBatch][k]
    ws += kAwqBatch * align256(a.k * 4);
    uint8_t *codes = ws;  // [kAwqBatch][n][k / 2]
    ws += kAwqBatch * align256(a.n * a.k / 2);
    float *scales = reinterpret_cast<float *>(ws);  // [kAwqBatch][n][k / group]
    ws += kAwqBatch * align256(meta);
    float *zeros = reinterpret_cast<float *>(ws);
    ws += kAwqBatch * align256(meta);
    double *partials = reinterpret_cast<double *>(ws);  // [kAwqBatch][blocks]
    // per-point strides in elements (every slot is a multiple of 256 bytes)
    const int64_t x_stride = align256(a.t * a.k * 2) / 2, s_stride = align256(a.k * 4) / 4;
    const int64_t code_stride = align256(a.n * a.k / 2), meta_stride = align256(meta) / 4;
    const int64_t blocks = w4a16_gemm_blocks(a.t, a.n);

    hipError_t e;
    if ((e = launch_gemm_bf16(a.x, a.w, a.t, a.n, a.k, y_ref, st)) != hipSuccess) return e;

    const uint32_t kblocks = (uint32_t)((a.k + 255) / 256);
    const int64_t x8 = a.t * a.k / 8;
    const uint32_t xblocks = (uint32_t)((x8 + 255) / 256 < 4096 ? (x8 + 255) / 256 : 4096);
    for (int i0 = 0; i0 <= a.n_grid; i0 += kAwqBatch) {
        const int points = a.n_grid + 1 - i0 < kAwqBatch ? a.n_grid + 1 - i0 : kAwqBatch;
        // the batch's scales and scaled activations, one launch each
        hipLaunchKernelGGL(awq_scale_kernel, dim3(kblocks, (uint32_t)points), dim3(256), 0, st, a.sx, (int)a.k, i0,
                           a.n_grid, s, s_stride);
        hipLaunchKernelGGL(div_act_kernel, dim3(xblocks, (uint32_t)points), dim3(256), 0, st, a.x, x8, (int)a.k, s,
                           s_stride, xa, x_stride);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // the batch's quantizations in one launch
        QuantArgs q{a.w, a.n, a.k, 4, a.symmetric, a.group, s, codes, scales, zeros};
        q.batch = points;
        q.cs_stride = s_stride;
        q.code_stride = code_stride;
        q.meta_stride = meta_stride;
        if ((e = launch_quantize(q, st)) != hipSuccess) return e;
        const WoArgs g{xa, a.t, codes, scales, zeros, a.n, a.k, a.symmetric, a.group, nullptr};
        if ((e = launch_w4a16_gemm_loss(g, points, x_stride, code_stride, meta_stride, y_ref, partials, st)) !=
            hipSuccess)
            return e;
        hipLaunchKernelGGL(loss_finish_kernel, dim3((uint32_t)points), dim3(256), 0, st, partials, blocks,
                           a.losses + i0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(awq_pick_kernel, dim3(kblocks), dim3(256), 0, st, a.losses, a.n_grid, a.sx, (int)a.k,
                       a.s_best, a.best);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const QuantArgs qb{a.w, a.n, a.k, 4, a.symmetric, a.group, a.s_best, a.codes, a.scales, a.zeros};
    return launch_quantize(qb, st);
}

}  // namespace lq
