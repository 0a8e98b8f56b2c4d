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
// MFMA operand fragment. A block of 4 waves computes 128 x 128 outputs (2 x 2
// waves of 64 x 64 = 4 x 4 tiles of 16 x 16) and walks k in 128-wide steps
// (32 MFMAs per wave between two barriers; 64-wide steps measured 3-26 %
// slower). The step's 128 x 128 slices of qx and qw go straight from memory
// into LDS (buffer loads with the LDS-write form, 16 bytes a lane), into a
// ring of kStages slots filled kStages - 1 steps ahead, so one wave per SIMD
// keeps several steps of loads in flight while its MFMAs run. No VGPRs hold
// staged data.
// LDS slot layout: 128 rows of 128 bytes per operand; the eight 16-byte
// chunks of row r are stored XOR-permuted by swz(r) = (r >> 1) & 7, so the 16
// rows read by one fragment load hit distinct banks.
// Blocks are mapped XCD-aware: the hardware deals block b to XCD b % 8, and
// the blocks that share a 128-row slice of qw are put on one XCD so the
// slice is fetched into that XCD's L2 once.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kStages = 4;                      // LDS ring depth (128 KB)
constexpr int kSlot = (BM + BN) * BK;           // bytes of one ring slot (qx rows, then qw rows)
constexpr int kLoadsPerStep = kSlot / 1024 / 4; // 1 KB loads per wave per step
// vmcnt limits (literals: they are pasted into the step barrier's asm)
#define kVmPrologue 16  // (kStages - 2) steps of loads may stay pending
#define kVmStep 8       // (kStages - 3) steps

LQ_DEVICE int swz(int r) { return (r >> 1) & 7; }

// s_waitcnt immediate (gfx9 layout): vmcnt(0), expcnt and lgkmcnt not waited on
constexpr int kWaitVm0 = 0x0F70;

#define LQ_STR2(x) #x
#define LQ_STR(x) LQ_STR2(x)

__global__ __launch_bounds__(256) void w8a8_kernel(const int8_t *__restrict__ qx, const float *__restrict__ sx,
                                                    int m, const int8_t *__restrict__ qw,
                                                    const float *__restrict__ sw, int n, int k,
                                                    int32_t *__restrict__ accout, float *__restrict__ y) {
    __shared__ __attribute__((aligned(1024))) int8_t ring[kStages][kSlot];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, kq = lane >> 4;

    // tile of this block
    const int nt = (n + BN - 1) / BN, mt = (m + BM - 1) / BM;
    int tn, tm;
    if ((nt & 7) == 0) {
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        tn = xcd * (nt >> 3) + idx / mt;
        tm = idx % mt;
    } else {
        tn = blockIdx.x % nt;
        tm = blockIdx.x / nt;
    }
    const int n0 = tn * BN, m0 = tm * BM;

    // rows past m (n) read zeros, or leave stale bytes, in LDS; they only
    // feed outputs that are never stored
    const int rows_m = min(BM, m - m0), rows_n = min(BN, n - n0);
    const auto ra = make_rsrc(qx + (int64_t)m0 * k, (uint32_t)rows_m * (uint32_t)k);
    const auto rb = make_rsrc(qw + (int64_t)n0 * k, (uint32_t)rows_n * (uint32_t)k);

    // This wave's loads: 1 KB pieces q = 8 wave + i (i < 8) of a slot; piece
    // q < 16 covers qx rows 8 q .. + 7, piece q >= 16 qw rows 8 (q - 16) ...
    // Lane l writes LDS bytes 16 l of the piece: row 8 q' + l / 8, chunk
    // slot l % 8, which holds the row's logical chunk (l % 8) ^ swz(row).
    uint32_t src_off[kLoadsPerStep];
#pragma unroll
    for (int i = 0; i < kLoadsPerStep; ++i) {
        const int q = kLoadsPerStep * wave + i;
        const int row = 8 * (q & 15) + (lane >> 3);
        src_off[i] = (uint32_t)row * (uint32_t)k + 16u * (uint32_t)((lane & 7) ^ swz(row));
    }
    const int nsteps = k / BK;
    auto issue = [&](int ks) {
        int8_t *slot = ring[ks % kStages];
        const bool in = ks < nsteps;  // later steps only keep the load count uniform
        // waves 0, 1 load qx pieces, waves 2, 3 qw pieces (wave-uniform branch);
        // plain cached loads: every qw slice is read by all m-blocks of its
        // XCD, so it must stay in L2
        if (wave < 2) {
#pragma unroll
            for (int i = 0; i < kLoadsPerStep; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (__attribute__((address_space(3))) void *)(slot + 1024 * (kLoadsPerStep * wave + i)), 16,
                    in ? src_off[i] + (uint32_t)ks * BK : kOutOfRange, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < kLoadsPerStep; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (__attribute__((address_space(3))) void *)(slot + 1024 * (kLoadsPerStep * wave + i)), 16,
                    in ? src_off[i] + (uint32_t)ks * BK : kOutOfRange, 0, 0, 0);
        }
    };

    i32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    // fragment addresses within a slot: lane (row l16, k quarter kq) of the
    // step's half h (64 k each)
    int a_off[2][4], b_off[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int ra_row = wm * 64 + t * 16 + l16, rb_row = wn * 64 + t * 16 + l16;
            a_off[h][t] = ra_row * BK + 16 * ((4 * h + kq) ^ swz(ra_row));
            b_off[h][t] = BM * BK + rb_row * BK + 16 * ((4 * h + kq) ^ swz(rb_row));
        }

    // The row and column scales of this lane's outputs, loaded up front
    // (rows past m and columns past n read zeros): the epilogue's stores then
    // never wait on a load. These loads precede every LDS-write load, so the
    // step waits below still count only the latter.
    const auto rsx = make_rsrc(sx + m0, (uint32_t)rows_m * 4);
    const auto rsw = make_rsrc(sw + n0, (uint32_t)rows_n * 4);
    float swc[4], sxr[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        swc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rsw, (uint32_t)(wn * 64 + j * 16 + l16) * 4, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sxr[i][v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rsx, (uint32_t)(wm * 64 + i * 16 + kq * 4 + v) * 4, 0, 0));
    auto read_frags = [&](int ks, i32x4 *af, i32x4 *bf) {
        const int8_t *slot = ring[ks % kStages];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[4 * h + t] = *reinterpret_cast<const i32x4 *>(slot + a_off[h][t]);
                bf[4 * h + t] = *reinterpret_cast<const i32x4 *>(slot + b_off[h][t]);
            }
    };
    auto mfmas = [&](const i32x4 *af, const i32x4 *bf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[4 * h + i], bf[4 * h + j], acc[i][j], 0, 0, 0);
    };
    // Step barrier. LDS-write loads are counted by vmcnt only and the
    // compiler does not track them, so the waits are explicit: a wave's own
    // loads of a step are done once at most N later loads are pending; after
    // the barrier every wave's are. No lgkmcnt wait: the only LDS reads of the
    // slot a step refills fed MFMAs of the step before, so they are complete,
    // and the next step's fragment reads stay in flight across the barrier.
#define LQ_STEP_SYNC(N) asm volatile("s_waitcnt vmcnt(" LQ_STR(N) ")\n\ts_barrier" ::: "memory")

    // Pipeline: step ks's fragments were read from LDS during step ks - 1, so
    // step ks reads step ks + 1's while its MFMAs run; the loads run
    // kStages - 1 steps ahead. Step ks's barrier certifies that step ks + 1
    // has landed and that every wave has finished step ks - 1, whose slot
    // (read during step ks - 2) the step's load then refills.
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    // With an odd step count the last iteration's second half computes the
    // step past the end, whose slot the out-of-range loads filled with zeros.
    i32x4 fa0[8], fb0[8], fa1[8], fb1[8];
    LQ_STEP_SYNC(kVmPrologue);
    read_frags(0, fa0, fb0);
    for (int ks = 0; ks < nsteps; ks += 2) {
        LQ_STEP_SYNC(kVmStep);
        issue(ks + kStages - 1);
        read_frags(ks + 1, fa1, fb1);
        mfmas(fa0, fb0);
        LQ_STEP_SYNC(kVmStep);
        issue(ks + kStages);
        read_frags(ks + 2, fa0, fb0);  // past the last step: read, never used
        mfmas(fa1, fb1);
    }
#undef LQ_STEP_SYNC
    // drain the trailing (out-of-range) loads and the scale loads; the
    // builtin (unlike an asm wait) tells the compiler nothing is pending, so
    // the guarded stores below carry no further waits
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // epilogue: lane holds acc[row 4 kq + v][col l16] of each tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + i * 16 + kq * 4 + v;
                if (row < m && col < n) {
                    const int32_t a = acc[i][j][v];
                    if (accout) accout[(int64_t)row * n + col] = a;
                    y[(int64_t)row * n + col] = ((float)a * sxr[i][v]) * swc[j];
                }
            }
    }
}
static_assert(kLoadsPerStep * (kStages - 2) == kVmPrologue && kLoadsPerStep * (kStages - 3) == kVmStep,
              "the vmcnt counts in the step barriers");

}  // namespace

hipError_t launch_w8a8_gemm(const W8Args &a, hipStream_t st) {
    const uint32_t blocks = (uint32_t)(((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM));
    hipLaunchKernelGGL(w8a8_kernel, dim3(blocks), dim3(256), 0, st, a.qx, a.sx, (int)a.m, a.qw, a.sw, (int)a.n, (int)a.k,
                       a.acc, a.y);
    return hipGetLastError();
}

}  // namespace lq
