// gemv_shared.hip -- decode GEMV at batch 4..16 on large matrices, for the
// three weight formats of the library, on v_mfma_f32_16x16x32_bf16 with
// every operand staged through LDS.
//
// Definitions:
//  * INT4 and INT8 ("LLM quantization deep dive", rainlib.com, W4A16 and the
//    W/A/KV notation's W8A16: integer weights dequantized inside the kernel
//    and multiplied with 16-bit activations, higher-precision accumulation):
//      y[b][r] = sum_j x[b][j] * (q[r][j] - z[r][j/G]) * s[r][j/G];
//  * MXFP4 ("3.6 Quantization", number-format table and "Granularity": FP4
//    E2M1 elements in blocks of 32 sharing one E8M0 power-of-two scale):
//      y[b][r] = sum_j x[b][j] * E2M1(c[r][j]) * 2^e[r][j/32].
//
// Why a separate kernel: at batch 4..16 the per-wave kernels re-read the
// activation fragment from L2 for every 16 or 32 rows, which at batch 16 is
// a third of the code traffic, and keep too few code bytes in flight per
// CU. Here a block of 4 waves works on kShRows = 128 rows together and
// shares each stage of k in LDS:
//  * a stage is 256 k of INT4 or MXFP4 codes or 128 k of INT8 codes: 128
//    bytes of every row either way, 16 KB per block;
//  * per stage every wave issues 4 of the block's 16 code loads (8 rows x
//    128 bytes each) and its share of the XR activation rows (XR = the batch
//    rounded up to 4, 8 or 16; rows past the batch read zeros), all as buffer
//    loads in the LDS-write form, so no operand passes through registers on
//    its way to LDS;
//  * scales and zeros come in windows of kWinSt (4, or 2 for INT4 at XR =
//    16) stages, double-buffered: at a window's first stage each wave loads
//    its quarter of the window, 4 bytes a lane with the lanes of a row
//    reading its consecutive entries (8 or 16 rows of 16-32 bytes per load).
//    Loading each stage's entries for the 128 rows instead costs a separate
//    cache line per lane; on the 70B shapes the windows take 10-16 % off
//    INT8 at batch 8-16, 2-21 % off MXFP4 and 5-14 % off INT4 on q|k|v,
//    gate|up and o at batch 4 (within a few per cent either way elsewhere);
//  * three slots: one stage is computed while the next is in flight. The
//    stage wait is the wave's own vmcnt (loads that write LDS are only
//    counted there) followed by a barrier; the slot refilled after it is the
//    one every wave finished before that barrier;
//  * wave w computes rows 32 w .. 32 w + 31 of the block as two 16-row MFMA
//    tiles that share the activation operand (A = 16 rows x 32 k of
//    weights, B = 32 k x 16 batch columns of activations; lane l serves
//    weight row and batch column l % 16 and k quarter l / 16).
// Weight operands, all exact in bf16:
//  * INT4: a nibble ORed into the mantissa of the bf16 128 gives 128 + q;
//    per 128-wide group the tile D_g and the activation sums X_g (an MFMA
//    against a bf16 ones operand) give acc += s (D_g - (128 + z) X_g)
//    (symmetric codes hold q + 8, so the constant is 136);
//  * INT8: v_cvt_f32_ubyte gives the byte's fp32 value, whose upper half is
//    its exact bf16; symmetric int8 codes are first turned into q + 128 by
//    an xor with 0x80, and acc += s (D_g - c X_g) with c = z or 128;
//  * MXFP4: v_cvt_scalef32_pk_bf16_fp4 with the block's scale 2^e converts
//    two codes into the exact bf16 values E2M1(c) 2^e (also where that is a
//    bf16 subnormal, and the MFMA keeps subnormal inputs), so the MFMAs
//    accumulate the output directly and no correction is needed. Each
//    lane's 32 k of a 16-byte code chunk are one block of 32.
// LDS layout of a slot: codes [128 rows][128 B], 16-byte chunk c of row r
// stored at c ^ ((r >> 1) & 7); activations [XR rows][2 x stage k bytes],
// chunk c of row r at c ^ r (batch column b reads row b % XR; columns past
// the batch are never stored). With these the 16 rows (columns) of one
// fragment read fall in distinct banks. The two window buffers follow the
// three slots in the same array: with the windows declared as an array of
// their own, the compiler made every wave wait for all of its outstanding
// LDS-write loads before each window read, which stalled the ring. At most
// 81,920 bytes, so 2 blocks fit a CU.
// With too few row blocks to fill the chip, k is split into runs of stages
// (blockIdx.y); the runs add their partial sums into y, zeroed first on the
// same stream, with float atomics, so with more than two runs the summation
// order (and the last bits of y) can differ from call to call. With one or
// two runs the result is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

constexpr int kShRows = 128;  // rows per block (32 per wave)
constexpr int kShSlots = 3;
constexpr uint32_t kShMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kShOnes = 0x3F803F80u;   // bf16 pair (1, 1)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <WeightFormat F>
struct ShFormat {
    static constexpr int kStageK = F == WeightFormat::kInt8 ? 128 : 256;  // k per stage (128 code bytes a row)
    static constexpr int kHalves = kStageK / 128;                         // 128-wide compute steps per stage
    static constexpr int kXRowBytes = 2 * kStageK;                        // activation bytes a row per stage
    static constexpr int kXChunks = kXRowBytes / 16;
    static constexpr int kXRowsPerPiece = 1024 / kXRowBytes;              // rows in a 1 KB load
    static constexpr int kMetaPerStage = F == WeightFormat::kInt8 ? 4 : 8;  // metadata bytes a row per stage
};

// Four code bytes u0..u3 -> bf16 pairs (u0, u1), (u2, u3): the byte-wise
// integer-to-float conversions select v_cvt_f32_ubyte{0..3}, and the upper
// half of an fp32 holding an integer below 256 is its exact bf16.
LQ_DEVICE void sh_bytes_to_bf16(uint32_t w, uint32_t &p01, uint32_t &p23) {
    const float f0 = (float)(w & 0xFFu);
    const float f1 = (float)((w >> 8) & 0xFFu);
    const float f2 = (float)((w >> 16) & 0xFFu);
    const float f3 = (float)(w >> 24);
    p01 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    p23 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// scales: fp32 [n][k / group] (INT4, INT8) or E8M0 bytes [n][k / 32] (MXFP4);
// zeros: fp32 [n][k / group] for asymmetric integer codes, else unused.
template <WeightFormat F, int XR, bool SYM, bool SPLIT>
__global__ __launch_bounds__(256) void gemv_shared_kernel(const uint16_t *__restrict__ x, int bsz,
                                                           const uint8_t *__restrict__ codes,
                                                           const void *__restrict__ scales,
                                                           const float *__restrict__ zeros, int n, int k,
                                                           int group, int stages_per_run, float *__restrict__ y) {
    using Fm = ShFormat<F>;
    // (the lambda below reads these copies: naming a static member of the
    // dependent type inside it drops the kernel from the host compilation)
    constexpr int kStageK = Fm::kStageK, kXRowBytes = Fm::kXRowBytes;
    constexpr bool kInt4 = F == WeightFormat::kInt4, kInt8 = F == WeightFormat::kInt8, kMx = F == WeightFormat::kMx;
    constexpr int kXPieces = XR * Fm::kXRowBytes / 1024;                  // 1 KB activation loads per stage
    constexpr int kXPerWave = kXPieces >= 4 ? kXPieces / 4 : 1;
    constexpr int kXOff = kShRows * 128, kDummy = kXOff + XR * Fm::kXRowBytes;
    constexpr int kSlot = kDummy + (kXPieces < 4 * kXPerWave ? 1024 : 0);  // a sink for waves without a piece
    // metadata windows: kWinSt stages of every row's scales (and zeros), two
    // buffers after the slots; 4-byte loads, kLpr lanes per row
    constexpr int kWinSt = kInt4 && XR == 16 ? 2 : 4;
    constexpr int kWinRow = kWinSt * Fm::kMetaPerStage;  // bytes a row per window and array
    constexpr int kArrays = kMx || SYM ? 1 : 2;           // scales, zeros
    constexpr int kWinBuf = kArrays * kShRows * kWinRow;
    constexpr int kWinOff = kShSlots * kSlot;
    constexpr int kLpr = kWinRow / 4, kRowsPerPiece = 64 / kLpr, kPiecesPerArr = kShRows / kRowsPerPiece;
    constexpr int kWinLoads = kArrays * kPiecesPerArr / 4;  // per wave, at a window's first stage
    constexpr int kVm = (kShSlots - 2) * (4 + kXPerWave);   // loads younger than the awaited stage
    static_assert(kXPerWave <= 2 && kWinOff + 2 * kWinBuf <= 80 * 1024 && XR * (kShRows + 1) * 4 <= kWinOff &&
                      kArrays * kPiecesPerArr % 4 == 0 && kWinSt >= kShSlots - 1,
                  "slot and window layout");
    // one array for slots and windows: the compiler makes a wave wait for all
    // of its LDS-write loads before reading a separately declared array
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kWinOff + 2 * kWinBuf];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    const int row0 = blockIdx.x * kShRows;
    const uint32_t row_bytes = kInt8 ? (uint32_t)k : (uint32_t)k / 2;
    const int nst = (k + Fm::kStageK - 1) / Fm::kStageK;
    const int s0 = blockIdx.y * stages_per_run;
    const int s1 = min(nst, s0 + stages_per_run);
    const int rows_here = min(kShRows, n - row0);
    // per-row metadata entries: groups (INT4, INT8) or scale bytes (MXFP4)
    // rows past n, k past the row and batch rows past bsz read zeros
    const auto rc = make_rsrc(codes + (int64_t)row0 * row_bytes, (uint32_t)rows_here * row_bytes);
    const auto rx = make_rsrc(x, (uint32_t)bsz * (uint32_t)k * 2);
    const int64_t meta_row = kMx ? k / 32 : k / group;  // entries a row
    const int meta_size = kMx ? 1 : 4;
    const auto rs = make_rsrc(static_cast<const uint8_t *>(scales) + row0 * meta_row * meta_size,
                              (uint32_t)(rows_here * meta_row * meta_size));
    const auto rz = make_rsrc(kMx || SYM ? static_cast<const float *>(nullptr) : zeros + row0 * meta_row,
                              kMx || SYM ? 0u : (uint32_t)(rows_here * meta_row) * 4);

    // code piece p = 4 wave + i: rows 8 p + lane / 8, stored chunk lane % 8
    uint32_t c_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        c_off[i] = (uint32_t)r * row_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    // activation piece q: rows kXRowsPerPiece q + lane / kXChunks, stored
    // chunk lane % kXChunks (fixed-size arrays: a lambda capturing an array
    // whose size depends on a template parameter is dropped from the host
    // compilation)
    uint32_t x_off[2];
    bool x_real[2];
#pragma unroll
    for (int i = 0; i < kXPerWave; ++i) {
        const int q = kXPerWave * wave + i;
        const int xr = Fm::kXRowsPerPiece * q + lane / Fm::kXChunks;
        x_real[i] = q < kXPieces;
        x_off[i] = (uint32_t)xr * (uint32_t)k * 2 + 16u * (uint32_t)((lane % Fm::kXChunks) ^ xr);
    }
    // A window holds, per row and array, one fp32 entry per 128-wide
    // half-stage (INT4, INT8: the scale or zero of the group the half lies
    // in; kLpr entries) or the E8M0 bytes of its stages (MXFP4, 8 a stage).
    // Layout of an array: INT4, INT8 [row / 4][entry][row % 4] (fp32), so the
    // four rows a lane's accumulators hold are one 16-byte read; MXFP4
    // [row][byte]. A 4-byte window load (piece p = kWinLoads wave + i, array
    // p / kPiecesPerArr, kRowsPerPiece rows) covers 256 contiguous LDS bytes;
    // lane l holds row rbase + 4 (l / (4 kLpr)) + l % 4, entry (l / 4) % kLpr
    // (INT4, INT8), or row rbase + l / kLpr, bytes 4 (l % kLpr) .. + 3 (MXFP4).
    const uint32_t meta_row_bytes = (uint32_t)((kMx ? k / 32 : k / group) * (kMx ? 1 : 4));
    const int w_row = kMx ? lane / kLpr : 4 * (lane / (4 * kLpr)) + lane % 4;  // row within the piece
    const int w_ent = kMx ? lane % kLpr : (lane / 4) % kLpr;                    // word within the row
    auto win_word = [&](int ws) -> uint32_t {  // this lane's byte in its row, window from stage ws
        return kMx ? (uint32_t)(ws * 8 + 4 * w_ent) : (uint32_t)(((ws * kStageK + 128 * w_ent) / group) * 4);
    };

    // Stages are visited in a rotated order: block b starts at window
    // b mod (windows of its run) and wraps around, so that the blocks do not
    // all read the same 128-byte column of their rows at once. INT4 and
    // MXFP4 only (70B gate|up, one run: INT4 2-3 %, MXFP4 8-15 % faster);
    // INT8 rows (k bytes apart rather than k / 2) measured 22 % slower with
    // it. Runs whose length is not a whole number of windows keep the
    // plain order. Slots and window buffers follow the visit index.
    constexpr bool kRotate = !kInt8;
    const int len = s1 - s0;
    int rot = 0;
    if (kRotate && len % kWinSt == 0 && len / kWinSt > 1) rot = (int)((blockIdx.x % (len / kWinSt)) * kWinSt);
    auto phys = [&](int iv) -> int {  // visit index -> stage (iv < len)
        int v = rot + iv;
        if (v >= len) v -= len;
        return s0 + v;
    };
    auto issue = [&](int iv) {
        uint8_t *slot = ring + (iv % kShSlots) * kSlot;
        const bool in = iv < len;
        const int st = in ? phys(iv) : s1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (__attribute__((address_space(3))) void *)(slot + 1024 * (4 * wave + i)), 16,
                in ? c_off[i] + (uint32_t)st * 128 : kOutOfRange, 0, 0, kNonTemporal);
#pragma unroll
        for (int i = 0; i < kXPerWave; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx,
                (__attribute__((address_space(3))) void *)(slot + (x_real[i] ? kXOff + 1024 * (kXPerWave * wave + i)
                                                                             : kDummy)),
                16, in && x_real[i] ? x_off[i] + (uint32_t)st * kXRowBytes : kOutOfRange, 0, 0, 0);
        if (iv % kWinSt == 0) {  // a window's first stage (wave-uniform)
            uint8_t *win = ring + kWinOff + ((iv / kWinSt) & 1) * kWinBuf;
            const uint32_t word = win_word(st);
#pragma unroll
            for (int i = 0; i < kWinLoads; ++i) {
                const int p = kWinLoads * wave + i;
                const int arr = p / kPiecesPerArr, rbase = kRowsPerPiece * (p % kPiecesPerArr);
                const int r = rbase + w_row;
                const uint32_t off = (uint32_t)r * meta_row_bytes + word;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    arr ? rz : rs, (__attribute__((address_space(3))) void *)(win + arr * kShRows * kWinRow + rbase * kWinRow),
                    4, in && r < rows_here ? off : kOutOfRange, 0, 0, 0);
            }
        }
    };

    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kShMagic));
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{kShOnes, kShOnes, kShOnes, kShOnes});
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // fragment reads. A: row 32 wave + 16 t + lane % 16; INT4 / MXFP4 chunk
    // 4 h + lane / 16 (its words j = 0..3 feed MFMA steps j), INT8 chunks
    // 2 (lane / 16) and 2 (lane / 16) + 1 (their word pairs feed the steps).
    // B: activation row (lane % 16) % XR, the 8 k that the lane's A holds in
    // step j: 16-byte piece 16 h + 4 (lane / 16) + j of the row.
    int a_off[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 32 * wave + 16 * t + l16;
            const int c = kInt8 ? 2 * kq + h : 4 * h + kq;
            a_off[t][h] = r * 128 + 16 * (c ^ ((r >> 1) & 7));
        }
    const int xrow = l16 % XR;
    int b_off[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b_off[h][j] = kXOff + xrow * Fm::kXRowBytes + 16 * ((16 * h + 4 * kq + j) ^ xrow);

#pragma unroll
    for (int i = 0; i < kShSlots - 1; ++i) issue(i);
    for (int iv = 0; iv < len; ++iv) {
        const int st = phys(iv);
        // stage st has landed for every wave; the slot refilled below was
        // last read in the previous iteration, before this barrier
        // (the next visited stage carries a window's loads when it starts one)
        if ((iv + 1) % kWinSt == 0)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVm + kWinLoads) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVm) : "memory");
        issue(iv + kShSlots - 1);
        const uint8_t *slot = ring + (iv % kShSlots) * kSlot;
        const int ws = st - iv % kWinSt;  // first stage of the window
        const uint8_t *win = ring + kWinOff + ((iv / kWinSt) & 1) * kWinBuf;
#pragma unroll
        for (int h = 0; h < Fm::kHalves; ++h) {
            // a half past the row's end (k a multiple of 128 only) is skipped:
            // its code and activation reads run into the next rows and its
            // window entries are the next row's
            if (st * kStageK + 128 * h >= k) break;
            bf16x8_t bop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bop[j] = *reinterpret_cast<const bf16x8_t *>(slot + b_off[h][j]);
            f32x4 xg = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (!kMx) {
#pragma unroll
                for (int j = 0; j < 4; ++j) xg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bop[j], xg, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8_t aop[4];
                if constexpr (kInt8) {
                    const u32x4 c0 = *reinterpret_cast<const u32x4 *>(slot + a_off[t][0]);
                    const u32x4 c1 = *reinterpret_cast<const u32x4 *>(slot + a_off[t][1]);
                    uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t p[4];
                        sh_bytes_to_bf16(SYM ? w[2 * j] ^ 0x80808080u : w[2 * j], p[0], p[1]);
                        sh_bytes_to_bf16(SYM ? w[2 * j + 1] ^ 0x80808080u : w[2 * j + 1], p[2], p[3]);
                        aop[j] = __builtin_bit_cast(bf16x8_t, u32x4{p[0], p[1], p[2], p[3]});
                    }
                } else {
                    const u32x4 cw = *reinterpret_cast<const u32x4 *>(slot + a_off[t][h]);
                    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
                    if constexpr (kInt4) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) aop[j] = __builtin_bit_cast(bf16x8_t, unpack_natural(w[j], magic));
                    } else {
                        // the lane's chunk is block 4 h + lane / 16 of the stage
                        const uint32_t e8 = win[kWinRow * (32 * wave + 16 * t + l16) + 8 * (st - ws) + 4 * h + kq];
                        const float scale = __uint_as_float(e8 << 23);  // 2^(e8 - 127); the byte 0 acts as 2^-127
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4 p;
                            p.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 0));
                            p.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 1));
                            p.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 2));
                            p.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 3));
                            aop[j] = __builtin_bit_cast(bf16x8_t, p);
                        }
                    }
                }
                if constexpr (kMx) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[j], bop[j], acc[t], 0, 0, 0);
                } else {
                    f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[j], bop[j], d, 0, 0, 0);
                    // D rows 4 (lane / 16) + v of the tile
                    const int rb = 32 * wave + 16 * t + 4 * kq;
                    // the half-stage's entries of rows rb .. rb + 3 in the window
                    const int eo = ((rb / 4) * kLpr + Fm::kHalves * (st - ws) + h) * 16;
                    const f32x4 sv = *reinterpret_cast<const f32x4 *>(win + eo);
                    f32x4 zv = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (!SYM) zv = *reinterpret_cast<const f32x4 *>(win + kShRows * kWinRow + eo);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float c = kInt4 ? (SYM ? 136.0f : 128.0f + zv[v]) : (SYM ? 128.0f : zv[v]);
                        acc[t][v] = __builtin_fmaf(sv[v], __builtin_fmaf(-c, xg[v], d[v]), acc[t][v]);
                    }
                }
            }
        }
    }
    // Output: transposed through the ring so that each store (or atomic) of
    // a wave covers 64 consecutive rows of one batch row -- 2 cache lines
    // instead of 16 -- which is what the atomics' cost depends on. Every
    // wave's loads, also the zero-filled ones issued past the last stage,
    // have landed before the ring is reused.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    constexpr int kOutStride = kShRows + 1;
    float *out = reinterpret_cast<float *>(ring);  // [XR][kOutStride]
    if (l16 < XR) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) out[l16 * kOutStride + 32 * wave + 16 * t + 4 * kq + v] = acc[t][v];
    }
    __syncthreads();
#pragma unroll
    for (int i = threadIdx.x; i < XR * kShRows; i += 256) {
        const int b = i / kShRows, r = i % kShRows;
        if (b < bsz && r < rows_here) {
            float *dst = y + (int64_t)b * n + row0 + r;
            if (SPLIT)
                atomicAdd(dst, out[b * kOutStride + r]);
            else
                *dst = out[b * kOutStride + r];
        }
    }
}

__global__ void gemv_zero_kernel(float *__restrict__ p, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0.0f;
}

// Runs of k (measured on MI355X). From 160 row blocks on, splitting gains
// at most a few per cent and often loses: one run. Below that a CU streams
// about the same bytes per second with one block as with two, so the time
// follows the busiest CU: T blocks take ceil(T / 256) rounds of one block
// per CU, and T = 258 costs about as much as 512. The run count (a power of
// two, at least 4 stages per run) maximises T / (256 ceil(T / 256)); a
// larger count has to win by more than 2 %.
constexpr int kCus = 256;

inline int pick_runs(int64_t blocks, int nst) {
    if (blocks >= 160) return 1;
    auto fill = [](int64_t t) { return (double)t / (double)(kCus * ((t + kCus - 1) / kCus)); };
    int best = 1;
    double best_fill = fill(blocks);
    for (int runs = 2; runs <= 64 && runs * 4 <= nst; runs *= 2) {
        const double f = fill(blocks * runs);
        if (f > best_fill + 0.02) {
            best = runs;
            best_fill = f;
        }
    }
    return best;
}

template <WeightFormat F, int XR, bool SYM>
hipError_t launch_xr(const SharedGemvArgs &a, hipStream_t st) {
    constexpr int kStageK = ShFormat<F>::kStageK;
    const int64_t blocks = (a.n + kShRows - 1) / kShRows;
    const int nst = (int)((a.k + kStageK - 1) / kStageK);
    const int runs = pick_runs(blocks, nst);
    const int per = (nst + runs - 1) / runs;
    const dim3 grid((uint32_t)blocks, (uint32_t)runs);
    if (runs > 1) {
        const int64_t count = a.m * a.n;
        hipLaunchKernelGGL(gemv_zero_kernel, dim3((uint32_t)((count + 255) / 256)), dim3(256), 0, st, a.y, count);
        hipLaunchKernelGGL((gemv_shared_kernel<F, XR, SYM, true>), grid, dim3(256), 0, st, a.x, (int)a.m, a.codes,
                           a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, per, a.y);
    } else {
        hipLaunchKernelGGL((gemv_shared_kernel<F, XR, SYM, false>), grid, dim3(256), 0, st, a.x, (int)a.m, a.codes,
                           a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, per, a.y);
    }
    return hipGetLastError();
}

template <WeightFormat F, bool SYM>
hipError_t launch_fmt(const SharedGemvArgs &a, hipStream_t st) {
    if (a.m <= 4) return launch_xr<F, 4, SYM>(a, st);
    if (a.m <= 8) return launch_xr<F, 8, SYM>(a, st);
    return launch_xr<F, 16, SYM>(a, st);
}

}  // namespace

// Where the shared-stage kernel beats the other kernels of its format
// (measured on MI355X over the 7B and 70B linears and ragged shapes):
//  INT4: batch 5..16 from about 40M weights (1.0-2.1x; below that the
//        LDS-ring kernel is faster), batch 4 from 40M weights where k >
//        8192 and from 64Mi weights otherwise (the VALU kernel: 8-19 %
//        faster on 6144 x 8192 and 12288 x 4096);
//  INT8: batch 4 from 40M weights with k >= 8192, 5..8 from 40M weights,
//        9..16 from 16M (1.1-2.9x);
//  MXFP4: batch 4..8 from 40M weights, 9..16 from 16M (1.1-4.9x).
// The block's codes (128 rows) and the activations are addressed with
// 32-bit offsets below 2^31.
bool shared_gemv_pays(WeightFormat f, int64_t m, int64_t n, int64_t k) {
    const int64_t row_bytes = f == WeightFormat::kInt8 ? k : k / 2;
    if (m < 4 || m > 16 || row_bytes * kShRows >= (int64_t(1) << 31) || m * k * 2 >= (int64_t(1) << 31))
        return false;
    const int64_t weights = n * k;
    const bool large = weights >= (int64_t(40) << 20), medium = weights >= (int64_t(16) << 20);
    switch (f) {
        // at batch 4 the VALU kernel stays ahead up to 64Mi weights with
        // k <= 8192 (12288 x 4096 symmetric: 10.2 against 12.5 us)
        case WeightFormat::kInt4: return m == 4 ? large && (k > 8192 || weights >= (int64_t(64) << 20)) : large;
        // INT8 at batch 4: ahead of the VALU kernel where k >= 8192 (70B
        // shapes 2-13 %, 4096 x 11008 14 %), behind at k = 4096 (12-17 %)
        case WeightFormat::kInt8: return m >= 9 ? medium : m >= 5 ? large : large && k >= 8192;
        case WeightFormat::kMx: return m >= 9 ? medium : large;
    }
    return false;
}

hipError_t launch_shared_gemv(WeightFormat f, const SharedGemvArgs &a, hipStream_t st) {
    if (a.m < 1 || a.m > 16) return hipErrorInvalidValue;
    switch (f) {
        case WeightFormat::kInt4:
            return a.symmetric ? launch_fmt<WeightFormat::kInt4, true>(a, st)
                               : launch_fmt<WeightFormat::kInt4, false>(a, st);
        case WeightFormat::kInt8:
            return a.symmetric ? launch_fmt<WeightFormat::kInt8, true>(a, st)
                               : launch_fmt<WeightFormat::kInt8, false>(a, st);
        case WeightFormat::kMx: return launch_fmt<WeightFormat::kMx, false>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace lq
