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
// Tiles: a block of 8 waves computes 128 x 256 outputs (2 x 4 waves of
// 64 x 64 = 4 x 4 MFMA tiles of 16 x 16) and walks k one 128-wide group per
// step. A step's 128 x 128 activation tile (32 KB) and the 256 columns' code
// words (16 KB) go straight from memory into one slot of an LDS ring (buffer
// loads with the LDS-write form, 16 bytes a lane), kStages - 1 steps ahead;
// so do the 256 columns' scales and zeros of the step's group (one 4-byte
// load form per wave: waves 0..3 scales, waves 4..7 zeros). Three slots of
// 50 KB leave room for one block per CU, i.e. two waves per SIMD, so one
// wave's unpacking and correction run while the other's MFMAs do (128 x 128
// blocks of 4 waves, one per SIMD: 22-29 % slower on the M = 2048 shapes).
// LDS slot layout: activation rows of 256 bytes whose sixteen 16-byte chunks
// are XOR-permuted by (row & 15), then code columns of 64 bytes whose four
// chunks are XOR-permuted by swz(col): the 16 rows (columns) read by one
// fragment load hit distinct banks.
// Blocks are mapped XCD-aware: the hardware deals block b to XCD b % 8, and
// the blocks that share a 256-column slice of the codes are put on one XCD.
//
// MXFP4 weights (gemm_mx_kernel; "3.6 Quantization", number-format table:
// FP4 E2M1 elements in blocks of 32 sharing an E8M0 power-of-two scale):
//   Y[m][n] = sum_j X[m][j] E2M1(c[n][j]) 2^e[n][j/32].
// The same tiles, ring and fragment layout; a lane's 32 k of a column in one
// step are exactly one block of 32, so v_cvt_scalef32_pk_bf16_fp4 with the
// block's 2^e turns each code byte into the exact bf16 pair E2M1(c) 2^e and
// the MFMAs accumulate Y directly: no zero point, no activation sums, no
// per-step correction. The step's 4 scale bytes of a column are one dword.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 256, GK = 128;  // block tile and group width
constexpr int kWaves = BN / 32;               // 2 x 4 waves of 64 x 64 outputs
constexpr int kStages = 3;                    // LDS ring depth
constexpr int kXBytes = BM * GK * 2;          // activation tile of a step
constexpr int kCBytes = BN * GK / 2;          // code tile of a step
constexpr int kSZOff = kXBytes + kCBytes;     // then 128 scales and 128 zeros (fp32)
constexpr int kSlot = kSZOff + 2 * BN * 4;
constexpr int kPiecesPerWave = (kXBytes + kCBytes) / 1024 / kWaves;  // 16-byte loads per wave per step
constexpr int kLoadsPerWave = kPiecesPerWave + 1;               // and one 4-byte load (scales or zeros)
// vmcnt literal pasted into the step barrier: (kStages - 2) steps of loads
#define LQ_GEMM_VM_STEP 7
static_assert(LQ_GEMM_VM_STEP == (kStages - 2) * kLoadsPerWave, "step barrier vmcnt");

constexpr uint32_t kMagicPair = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kOnePair = 0x3F803F80u;    // bf16 pair (1, 1)
// s_waitcnt immediate (gfx9 layout): vmcnt(0), expcnt and lgkmcnt not waited on
constexpr int kWaitVm0 = 0x0F70;

#define LQ_GEMM_STR2(x) #x
#define LQ_GEMM_STR(x) LQ_GEMM_STR2(x)

LQ_DEVICE int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Several products of the same shape in one launch (the AWQ grid points):
// blockIdx.y selects one, whose operands sit at the given element strides
// from the first. LOSS: instead of storing y, the block adds up
// (yref - y)^2 over its outputs in fp64 (lane order, then the waves in a
// fixed order) and writes the sum to loss[blockIdx.y * gridDim.x + blockIdx.x].
struct GemmBatch {
    int64_t x_stride, code_stride, meta_stride;
    const float *yref;
    double *loss;
};

template <bool SYM, bool LOSS>
__global__ __launch_bounds__(512) void gemm_w4_kernel(const uint16_t *__restrict__ x, int m, int n, int k,
                                                       const uint8_t *__restrict__ codes,
                                                       const float *__restrict__ scales,
                                                       const float *__restrict__ zeros, int group,
                                                       float *__restrict__ y, GemmBatch batch) {
    // the only LDS array (with a second one declared, the compiler waits for
    // all of a wave's LDS-write loads before every fragment read); the loss
    // epilogue reuses its first bytes
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][kSlot];
    x += (int64_t)blockIdx.y * batch.x_stride;
    codes += (int64_t)blockIdx.y * batch.code_stride;
    scales += (int64_t)blockIdx.y * batch.meta_stride;
    if (!SYM) zeros += (int64_t)blockIdx.y * batch.meta_stride;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int l16 = lane & 15, kq = lane >> 4;

    // tile of this block
    const int nt_count = (n + BN - 1) / BN, mt_count = (m + BM - 1) / BM;
    int tn, tm;
    if ((nt_count & 7) == 0) {
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        tn = xcd * (nt_count >> 3) + idx / mt_count;
        tm = idx % mt_count;
    } else {
        tn = blockIdx.x % nt_count;
        tm = blockIdx.x / nt_count;
    }
    const int n0 = tn * BN, m0 = tm * BM;
    const int ng = k / group;
    const int ngroups = k / GK;

    // rows past m and code columns past n read zeros, or leave stale bytes,
    // in LDS; they only feed outputs that are never stored
    const int rows_m = min(BM, m - m0), rows_n = min(BN, n - n0);
    const uint32_t row_bytes = (uint32_t)k / 2;
    const auto rx = make_rsrc(x + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k * 2);
    const auto rc = make_rsrc(codes + (int64_t)n0 * row_bytes, (uint32_t)rows_n * row_bytes);
    const auto rs = make_rsrc(scales + (int64_t)n0 * ng, (uint32_t)rows_n * ng * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)n0 * ng, SYM ? 0u : (uint32_t)rows_n * ng * 4);

    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagicPair));
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{kOnePair, kOnePair, kOnePair, kOnePair});

    // This wave's loads: 1 KB pieces q = kPiecesPerWave * wave + i of a slot.
    // Pieces 0..31: activation rows 4 q .. + 3; lane l writes LDS bytes 16 l
    // of the piece: row 4 q + l / 16, chunk slot l % 16, holding the row's
    // logical chunk (l % 16) ^ (row & 15). Pieces 32..39: code columns
    // 16 p .. + 15 (p = q - 32); lane l: column 16 p + l / 4, chunk slot l % 4,
    // holding logical chunk (l % 4) ^ swz(column).
    uint32_t src_off[kPiecesPerWave];
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) {
        const int q = kPiecesPerWave * wave + i;
        if (q < kXBytes / 1024) {
            const int row = 4 * q + (lane >> 4);
            src_off[i] = (uint32_t)row * (uint32_t)k * 2 + 16u * (uint32_t)((lane & 15) ^ (row & 15));
        } else {
            const int col = 16 * (q - kXBytes / 1024) + (lane >> 2);
            src_off[i] = (uint32_t)col * row_bytes + 16u * (uint32_t)((lane & 3) ^ swz(col));
        }
    }
    auto issue = [&](int g) {
        uint8_t *slot = ring[g % kStages];
        const bool in = g < ngroups;  // later steps only keep the load count uniform
#pragma unroll
        for (int i = 0; i < kPiecesPerWave; ++i) {
            const int q = kPiecesPerWave * wave + i;
            const bool is_x = q < kXBytes / 1024;  // wave-uniform
            const uint32_t step_bytes = is_x ? GK * 2 : GK / 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_x ? rx : rc,
                                                     (__attribute__((address_space(3))) void *)(slot + 1024 * q), 16,
                                                     in ? src_off[i] + (uint32_t)g * step_bytes : kOutOfRange, 0, 0,
                                                     0);
        }
        // scales (waves 0..3) or zeros (waves 4..7) of the group, columns
        // 64 (wave & 3) + lane; no zeros when symmetric: an empty range
        const uint32_t gi = (uint32_t)((g * GK) / group);
        const uint32_t so = (uint32_t)((64 * (wave & 3) + lane) * ng) * 4 + gi * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 4 ? rs : rz,
                                                 (__attribute__((address_space(3))) void *)(slot + kSZOff + 256 * wave),
                                                 4, in ? so : kOutOfRange, 0, 0, 0);
    };

    // fragment addresses within a slot
    int a_off[4][4], c_off[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)  // lane's k = 32 kq + 8 j + [0, 8): logical chunk 4 kq + j
            a_off[mt][j] = (wm * 64 + mt * 16 + l16) * (GK * 2) + 16 * ((4 * kq + j) ^ l16);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int col = wn * 64 + nt * 16 + l16;
        c_off[nt] = kXBytes + col * (GK / 2) + 16 * (kq ^ swz(col));
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    for (int g = 0; g < ngroups; ++g) {
        // Step barrier. LDS-write loads are counted by vmcnt only and the
        // compiler does not track them, so the wait is explicit: this wave's
        // loads of step g are done once at most (kStages - 2) steps' loads
        // are younger; after the barrier every wave's are, and every wave has
        // finished step g - 1, whose slot the issue below refills.
        asm volatile("s_waitcnt vmcnt(" LQ_GEMM_STR(LQ_GEMM_VM_STEP) ")\n\ts_barrier" ::: "memory");
        issue(g + kStages - 1);

        const uint8_t *slot = ring[g % kStages];
        // scales and zeros of columns wn*64 + nt*16 + l16
        float sc[4], zc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int col = wn * 64 + nt * 16 + l16;
            sc[nt] = reinterpret_cast<const float *>(slot + kSZOff)[col];
            zc[nt] = SYM ? 0.0f : reinterpret_cast<const float *>(slot + kSZOff + BN * 4)[col];
        }
        u32x4 cw[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) cw[nt] = *reinterpret_cast<const u32x4 *>(slot + c_off[nt]);
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
                const bf16x8_t aop = *reinterpret_cast<const bf16x8_t *>(slot + a_off[mt][j]);
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
    }
    // drain the trailing (out-of-range) LDS-write loads before the block
    // exits; the builtin also tells the compiler nothing is pending
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // epilogue: lane holds Y[row 4 kq + v][col l16] of each 16 x 16 tile
    if constexpr (LOSS) {
        // all 64 reference loads first (outputs past m or n read element 0
        // and are skipped below): loads under per-output branches were each
        // waited for in turn, about 40 us per workgroup
        float yr[4][4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = m0 + wm * 64 + mt * 16 + kq * 4 + v;
                    const int col = n0 + wn * 64 + nt * 16 + l16;
                    yr[mt][nt][v] = batch.yref[row < m && col < n ? (int64_t)row * n + col : 0];
                }
        double sq = 0.0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = m0 + wm * 64 + mt * 16 + kq * 4 + v;
                    const int col = n0 + wn * 64 + nt * 16 + l16;
                    const double d = (double)yr[mt][nt][v] - (double)acc[mt][nt][v];
                    if (row < m && col < n) sq = __builtin_fma(d, d, sq);
                }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
        // every wave's trailing loads have landed (each waited for its own
        // above) and no wave reads the ring any more past this barrier
        __syncthreads();
        double *wave_loss = reinterpret_cast<double *>(&ring[0][0]);
        if (lane == 0) wave_loss[wave] = sq;
        __syncthreads();
        if (tid == 0)
            batch.loss[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] =
                ((((((wave_loss[0] + wave_loss[1]) + wave_loss[2]) + wave_loss[3]) + wave_loss[4]) + wave_loss[5]) +
                 wave_loss[6]) +
                wave_loss[7];
    } else {
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
}

__global__ __launch_bounds__(512) void gemm_mx_kernel(const uint16_t *__restrict__ x, int m, int n, int k,
                                                      const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, float *__restrict__ y) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][kSlot];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int l16 = lane & 15, kq = lane >> 4;

    const int nt_count = (n + BN - 1) / BN, mt_count = (m + BM - 1) / BM;
    int tn, tm;
    if ((nt_count & 7) == 0) {
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        tn = xcd * (nt_count >> 3) + idx / mt_count;
        tm = idx % mt_count;
    } else {
        tn = blockIdx.x % nt_count;
        tm = blockIdx.x / nt_count;
    }
    const int n0 = tn * BN, m0 = tm * BM;
    const int ngroups = k / GK;
    const uint32_t srow = (uint32_t)k / 32;  // scale bytes per row

    const int rows_m = min(BM, m - m0), rows_n = min(BN, n - n0);
    const uint32_t row_bytes = (uint32_t)k / 2;
    const auto rx = make_rsrc(x + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k * 2);
    const auto rc = make_rsrc(codes + (int64_t)n0 * row_bytes, (uint32_t)rows_n * row_bytes);
    const auto rs = make_rsrc(scales + (int64_t)n0 * srow, (uint32_t)rows_n * srow);

    // the same 1 KB pieces as the INT4 kernel (activation rows, code columns)
    uint32_t src_off[kPiecesPerWave];
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) {
        const int q = kPiecesPerWave * wave + i;
        if (q < kXBytes / 1024) {
            const int row = 4 * q + (lane >> 4);
            src_off[i] = (uint32_t)row * (uint32_t)k * 2 + 16u * (uint32_t)((lane & 15) ^ (row & 15));
        } else {
            const int col = 16 * (q - kXBytes / 1024) + (lane >> 2);
            src_off[i] = (uint32_t)col * row_bytes + 16u * (uint32_t)((lane & 3) ^ swz(col));
        }
    }
    auto issue = [&](int g) {
        uint8_t *slot = ring[g % kStages];
        const bool in = g < ngroups;
#pragma unroll
        for (int i = 0; i < kPiecesPerWave; ++i) {
            const int q = kPiecesPerWave * wave + i;
            const bool is_x = q < kXBytes / 1024;
            const uint32_t step_bytes = is_x ? GK * 2 : GK / 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_x ? rx : rc,
                                                     (__attribute__((address_space(3))) void *)(slot + 1024 * q), 16,
                                                     in ? src_off[i] + (uint32_t)g * step_bytes : kOutOfRange, 0, 0,
                                                     0);
        }
        // the step's 4 scale bytes of columns 64 (wave & 3) + lane (waves 0..3);
        // waves 4..7 issue an empty load so every wave counts the same loads
        const uint32_t so = (uint32_t)(64 * (wave & 3) + lane) * srow + (uint32_t)g * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(slot + kSZOff + 256 * wave),
                                                 4, in && wave < 4 ? so : kOutOfRange, 0, 0, 0);
    };

    int a_off[4][4], c_off[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            a_off[mt][j] = (wm * 64 + mt * 16 + l16) * (GK * 2) + 16 * ((4 * kq + j) ^ l16);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int col = wn * 64 + nt * 16 + l16;
        c_off[nt] = kXBytes + col * (GK / 2) + 16 * (kq ^ swz(col));
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    for (int g = 0; g < ngroups; ++g) {
        asm volatile("s_waitcnt vmcnt(" LQ_GEMM_STR(LQ_GEMM_VM_STEP) ")\n\ts_barrier" ::: "memory");
        issue(g + kStages - 1);

        const uint8_t *slot = ring[g % kStages];
        // this lane's block of 32 in column col is block kq of the step:
        // 2^(e - 127) from the E8M0 byte in the fp32 exponent field (the
        // byte 0, +0.0f, acts as 2^-127 in the scaled conversion)
        float scale[4];
        u32x4 cw[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int col = wn * 64 + nt * 16 + l16;
            const uint32_t e8 = slot[kSZOff + 256 * (col >> 6) + 4 * (col & 63) + kq];
            scale[nt] = __uint_as_float(e8 << 23);
            cw[nt] = *reinterpret_cast<const u32x4 *>(slot + c_off[nt]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8_t bop[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t w = j == 0 ? cw[nt].x : j == 1 ? cw[nt].y : j == 2 ? cw[nt].z : cw[nt].w;
                u32x4 p;
                p.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale[nt], 0));
                p.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale[nt], 1));
                p.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale[nt], 2));
                p.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale[nt], 3));
                bop[nt] = __builtin_bit_cast(bf16x8_t, p);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8_t aop = *reinterpret_cast<const bf16x8_t *>(slot + a_off[mt][j]);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[nt], acc[mt][nt], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
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

hipError_t launch_mxfp4_gemm(const MxArgs &a, hipStream_t st) {
    const uint32_t blocks = (uint32_t)(((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_mx_kernel, dim3(blocks), dim3(512), 0, st, a.x, (int)a.m, (int)a.n, (int)a.k, a.codes,
                       a.scales, a.y);
    return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const WoArgs &a, hipStream_t st) {
    const uint32_t blocks = (uint32_t)(((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM));
    const GemmBatch one{0, 0, 0, nullptr, nullptr};
    if (a.symmetric)
        hipLaunchKernelGGL((gemm_w4_kernel<true, false>), dim3(blocks), dim3(512), 0, st, a.x, (int)a.m, (int)a.n,
                           (int)a.k, a.codes, a.scales, a.zeros, (int)a.group, a.y, one);
    else
        hipLaunchKernelGGL((gemm_w4_kernel<false, false>), dim3(blocks), dim3(512), 0, st, a.x, (int)a.m, (int)a.n,
                           (int)a.k, a.codes, a.scales, a.zeros, (int)a.group, a.y, one);
    return hipGetLastError();
}

int64_t w4a16_gemm_blocks(int64_t m, int64_t n) { return ((n + BN - 1) / BN) * ((m + BM - 1) / BM); }

hipError_t launch_w4a16_gemm_loss(const WoArgs &a, int points, int64_t x_stride, int64_t code_stride,
                                  int64_t meta_stride, const float *yref, double *loss, hipStream_t st) {
    const uint32_t blocks = (uint32_t)w4a16_gemm_blocks(a.m, a.n);
    const GemmBatch b{x_stride, code_stride, meta_stride, yref, loss};
    if (a.symmetric)
        hipLaunchKernelGGL((gemm_w4_kernel<true, true>), dim3(blocks, (uint32_t)points), dim3(512), 0, st, a.x,
                           (int)a.m, (int)a.n, (int)a.k, a.codes, a.scales, a.zeros, (int)a.group, a.y, b);
    else
        hipLaunchKernelGGL((gemm_w4_kernel<false, true>), dim3(blocks, (uint32_t)points), dim3(512), 0, st, a.x,
                           (int)a.m, (int)a.n, (int)a.k, a.codes, a.scales, a.zeros, (int)a.group, a.y, b);
    return hipGetLastError();
}

}  // namespace lq
