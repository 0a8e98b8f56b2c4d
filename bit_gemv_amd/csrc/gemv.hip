// gemv.hip -- W4A16 decode GEMV for gfx950: a VALU (v_dot2_f32_bf16) kernel
// for batch 1..4 and MFMA (16x16x32 bf16) kernels for batch 5..16.
//
// Definition ("LLM quantization deep dive", rainlib.com, W4A16: INT4 weights
// in memory, unpacked and dequantized inside the kernel and multiplied with
// 16-bit activations, higher-precision accumulation):
//   y[b][r] = sum_j x[b][j] * (q[r][j] - z[r][j/G]) * s[r][j/G].
// At small batch the product is bound by the bytes of codes and scales
// streamed from HBM ("3.6 Quantization": batch-1 decode time is bytes read
// over bandwidth), so the kernels are built around coalesced 16-byte code
// loads kept in flight and a small VALU budget per weight:
//
//  * A nibble c ORed into the mantissa of the bf16 0x4300 (= 128) gives the
//    bf16 value 128 + c exactly, so one v_and_or_b32 turns two nibbles of a
//    code word into a packed bf16 pair. Products with bf16 activations are
//    exact in fp32.
//  * The offset and the zero point are folded into a per-group correction:
//    sum x (q - z) s = s * (sum x (128 + q) - (128 + z) * sum x), with the
//    activation sum formed once per activation segment.
//  * Nibbles 0..3 of a code word pair with nibbles 4..7, so activations are
//    re-paired (x0, x4), (x1, x5), ... when loaded.
// Partial sums are reduced with butterflies inside a wave and through LDS
// across waves; no atomics, so results are deterministic. Batch 4..16 on
// large matrices goes to the shared-stage kernel of gemv_shared.hip instead.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kNib = 0x000F000Fu;
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)
constexpr int kChunk = 2048;              // k covered by one wave-wide 16-byte load

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 8 consecutive bf16 activations [x0 x1][x2 x3][x4 x5][x6 x7] -> pairs in
// the order the nibble extraction produces: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
LQ_DEVICE void pair_x(const u32x4 v, uint32_t *p) {
    p[0] = (v.x & 0xFFFFu) | (v.z << 16);
    p[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p[2] = (v.y & 0xFFFFu) | (v.w << 16);
    p[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
}

// Code word (element i of 8 at bits 4i..4i+3) -> 4 bf16 pairs (128 + c_i,
// 128 + c_{i+4}), i = 0..3. `magic` holds kMagic (passed in a VGPR).
LQ_DEVICE void unpack_word(uint32_t w, uint32_t *p, uint32_t magic) {
    p[0] = (w & kNib) | magic;
    p[1] = ((w >> 4) & kNib) | magic;
    p[2] = ((w >> 8) & kNib) | magic;
    p[3] = ((w >> 12) & kNib) | magic;
}

LQ_DEVICE float dot8(uint32_t w, const uint32_t *xp, float acc, uint32_t magic) {
    uint32_t p[4];
    unpack_word(w, p, magic);
    acc = dot2_bf16(p[0], xp[0], acc);
    acc = dot2_bf16(p[1], xp[1], acc);
    acc = dot2_bf16(p[2], xp[2], acc);
    acc = dot2_bf16(p[3], xp[3], acc);
    return acc;
}

// ---------------------------------------------------------------------------
// VALU kernel, batch B <= 4.
// Block = WPB waves (4, or 8 for an eight-way k split). The waves split the
// 2048-wide chunks of k (ks_count ways) and the block's rows (WPB / ks_count
// row sets of RW rows). For each chunk a
// wave first loads and pairs its 32 activations per batch row (L2 hits),
// then issues the 16-byte code loads (and scales, zeros) of all RW rows
// through buffer resources that cover only its rows, so rows past n and
// lanes past k read zeros instead of needing branches; then it computes as
// rows arrive. Per-row partial sums stay in registers until one transposed
// reduction at the end.
// ---------------------------------------------------------------------------
// G128: group == 128 and k a multiple of 512. Then all scales (and zeros) a wave needs for one chunk
// -- RW rows x 16 groups -- come from a single 16-byte load per lane (lanes
// 0..4RW-1 scales, the next 4RW lanes zeros), are transposed through the
// wave's own LDS slice and read back four rows per ds_read_b128. Per-row
// 4-byte loads would otherwise be 2 RW of the wave's vector-memory
// instructions per chunk, and instruction issue, not bytes, bounds the
// kernel at that point.
template <int B, int RW, bool SYM, bool G128, int WPB>
__global__ __launch_bounds__(WPB * 64) void gemv_valu_kernel(const uint16_t *__restrict__ x,
                                                              const uint8_t *__restrict__ codes,
                                                              const float *__restrict__ scales,
                                                              const float *__restrict__ zeros, int n, int k,
                                                              int group, int ks_count, float *__restrict__ y) {
    static_assert(!G128 || RW == 4 || RW == 8, "scale staging assumes 4 or 8 rows per wave");
    static_assert(WPB == 4 || WPB == 8, "waves per block");
    __shared__ float red[WPB][B][RW];
    __shared__ __attribute__((aligned(16))) float sz_lds[G128 ? WPB : 1][2][16][RW];
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) so the buffer resources below live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // ks_count is a power of two up to WPB
    const int ks_log = __builtin_ctz((unsigned)ks_count);
    const int ks = wave & (ks_count - 1);
    const int rs = wave >> ks_log;
    const int row0 = (blockIdx.x * (WPB >> ks_log) + rs) * RW;
    const int ng = k / group;
    const int nchunks = (k + kChunk - 1) / kChunk;
    const uint32_t row_bytes = (uint32_t)k / 2;
    const int rows_here = row0 < n ? min(RW, n - row0) : 0;
    const auto rc = make_rsrc(codes + (int64_t)row0 * row_bytes, rows_here * row_bytes);
    const auto rsc = make_rsrc(scales + (int64_t)row0 * ng, rows_here * ng * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)row0 * ng, SYM ? 0 : rows_here * ng * 4);
    // 0x43004300 in a VGPR so the nibble extraction selects v_and_or_b32
    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));

    float acc[B][RW];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[b][r] = 0.0f;

    for (int c = ks; c < nchunks; c += ks_count) {
        const int k0 = c * kChunk + lane * 32;
        const bool kv = k0 < k;
        // All loads of the chunk first: activations (L2 hits), then codes,
        // scales and zeros of every row; nothing waits until all are issued.
        u32x4 xv[B][4];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const auto rx = make_rsrc(x + (int64_t)b * k, (uint32_t)k * 2);
            const uint32_t xo = kv ? (uint32_t)k0 * 2 : kOutOfRange;
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[b][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * j, 0, 0);
        }
        const uint32_t co = kv ? (uint32_t)k0 / 2 : kOutOfRange;
        u32x4 cw[RW];
        float sc[RW], zc[RW];
        u32x4 szv;  // G128: this lane's four scales or zeros of one row
        if (G128) {
            // lane L < 4 RW: scales of row L / 4, groups 4 (L % 4) .. + 3 of the
            // chunk; lanes 4 RW .. 8 RW - 1: the same for zeros
            const int which = lane / (4 * RW), lr = lane % (4 * RW);
            const int g0 = c * (kChunk / 128) + 4 * (lr & 3);
            const uint32_t off = g0 < ng ? (uint32_t)((lr >> 2) * ng + g0) * 4 : kOutOfRange;
            // two loads with wave-uniform descriptors; the other lanes read zeros
            const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rsc, which == 0 ? off : kOutOfRange, 0, 0);
            const u32x4 zv = SYM ? u32x4{0u, 0u, 0u, 0u}
                                 : __builtin_amdgcn_raw_buffer_load_b128(rz, which == 1 ? off : kOutOfRange, 0, 0);
            szv = which == 0 ? sv : zv;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r)
            cw[r] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + r * row_bytes, 0, kNonTemporal);
        if (!G128) {
            const uint32_t so = kv ? (uint32_t)(k0 / group) * 4 : kOutOfRange;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                sc[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, so + r * ng * 4, 0, 0));
                zc[r] = SYM ? 0.0f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, so + r * ng * 4, 0, 0));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (G128) {
            // transpose through LDS: [which][group in chunk][row]
            const int which = lane / (4 * RW), lr = lane % (4 * RW);
            if (which < 2) {
                // (__uint_as_float, not __builtin_bit_cast: this clang reads a
                // bit-cast vector element from the vector's first element)
                const int gg = 4 * (lr & 3), rr = lr >> 2;
                sz_lds[wave][which][gg + 0][rr] = __uint_as_float(szv.x);
                sz_lds[wave][which][gg + 1][rr] = __uint_as_float(szv.y);
                sz_lds[wave][which][gg + 2][rr] = __uint_as_float(szv.z);
                sz_lds[wave][which][gg + 3][rr] = __uint_as_float(szv.w);
            }
            // the writes above and reads below are in one wave: LDS executes a
            // wave's operations in order; keep the compiler from reordering
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int gl = lane >> 2;            // group of this lane's 32 k within the chunk
#pragma unroll
            for (int r4 = 0; r4 < RW; r4 += 4) {
                const f32x4 sv = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][0][gl][r4]);
                sc[r4] = sv.x; sc[r4 + 1] = sv.y; sc[r4 + 2] = sv.z; sc[r4 + 3] = sv.w;
                if (!SYM) {
                    const f32x4 zv = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][1][gl][r4]);
                    zc[r4] = zv.x; zc[r4 + 1] = zv.y; zc[r4 + 2] = zv.z; zc[r4 + 3] = zv.w;
                } else {
                    zc[r4] = zc[r4 + 1] = zc[r4 + 2] = zc[r4 + 3] = 0.0f;
                }
            }
        }
        uint32_t xp[B][16];
        float xs[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) pair_x(xv[b][j], &xp[b][4 * j]);
            xs[b] = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) xs[b] = dot2_bf16(xp[b][j], kOnes, xs[b]);
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            sc[r] = kv ? sc[r] : 0.0f;
            zc[r] = SYM ? 136.0f : 128.0f + zc[r];
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float d = 0.0f;
                d = dot8(cw[r].x, &xp[b][0], d, magic);
                d = dot8(cw[r].y, &xp[b][4], d, magic);
                d = dot8(cw[r].z, &xp[b][8], d, magic);
                d = dot8(cw[r].w, &xp[b][12], d, magic);
                acc[b][r] = __builtin_fmaf(sc[r], __builtin_fmaf(-zc[r], xs[b], d), acc[b][r]);
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
        if (row < n) y[(int64_t)b * n + row] = v;
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel, batch 5..16 (v_mfma_f32_16x16x32_bf16).
// A = weights (16 rows x 32 k), B = activations (32 k x 16 batch columns),
// D = 16 rows x 16 columns in fp32. Lane l serves weight row l % 16 (A) and
// batch column l % 16 (B), k quarter l / 16: its 16-byte code load covers 32
// consecutive k of a 128-wide group, MFMA step j (0..3) takes code word j
// unpacked in natural k order, and the activation operand of step j is the
// lane's 8 consecutive bf16 at the same k; the four steps cover the group.
// Per group the tile D_g and the activation sums X_g (an MFMA against a
// bf16 ones operand, which lands in the same layout) give
// acc += s (D_g - (128 + z) X_g). Columns past the batch read a valid batch
// row and are never stored.
// A wave owns two row tiles (32 rows, sharing the activation operand) and a
// contiguous run of gpw groups; the block's waves (up to 16) split k and
// reduce through LDS. Each group's scales and zeros of the 32 rows come from
// one 4-byte load per lane and are transposed through the wave's LDS slice.
// The next group's loads are issued before the current group is computed.
// ---------------------------------------------------------------------------
constexpr int kMfmaRows = 32;  // rows per block (and per wave)

template <bool SYM>
__global__ __launch_bounds__(1024) void gemv_mfma_kernel(const uint16_t *__restrict__ x, int bsz,
                                                          const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ scales,
                                                          const float *__restrict__ zeros, int n, int k,
                                                          int group, int gpw, float *__restrict__ y) {
    __shared__ float red[16][2][16][17];
    __shared__ __attribute__((aligned(16))) float sz_lds[16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    const int row0 = blockIdx.x * kMfmaRows;
    const int ng = k / group;
    const int ng128 = k / 128;
    const uint32_t row_bytes = (uint32_t)k / 2;
    const int rows_here = min(kMfmaRows, n - row0);
    // one code descriptor per 16-row tile (rows past n read zeros)
    const auto rc0 = make_rsrc(codes + (int64_t)row0 * row_bytes, (uint32_t)min(16, rows_here) * row_bytes);
    const auto rc1 = make_rsrc(codes + (int64_t)(row0 + 16) * row_bytes,
                               (uint32_t)max(0, rows_here - 16) * row_bytes);
    const auto rsc = make_rsrc(scales + (int64_t)row0 * ng, (uint32_t)rows_here * ng * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)row0 * ng, SYM ? 0u : (uint32_t)rows_here * ng * 4);
    // activation row of this lane's batch column (columns past the batch
    // reuse a valid row; their outputs are dropped)
    const uint16_t *xrow = x + (int64_t)min(l16, bsz - 1) * k + 32 * kq;
    const int g_begin = wave * gpw, g_end = min(ng128, g_begin + gpw);
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{kOnes, kOnes, kOnes, kOnes});
    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));

    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    struct GroupLoads {
        u32x4 cw0, cw1, xv[4];
        float sz;
    };
    // loads of group g; past this wave's run the addresses are clamped to its
    // last group and the scales read zero, so such a group adds nothing
    auto issue = [&](int g, GroupLoads &L) {
        const bool gv = g < g_end;
        g = min(g, g_end - 1);
        const uint32_t co = (uint32_t)l16 * row_bytes + (uint32_t)g * 64 + 16u * kq;
        L.cw0 = __builtin_amdgcn_raw_buffer_load_b128(rc0, co, 0, kNonTemporal);
        L.cw1 = __builtin_amdgcn_raw_buffer_load_b128(rc1, co, 0, kNonTemporal);
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(xrow + (int64_t)g * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j) L.xv[j] = xp[j];
        // lanes 0..31: scale of row lane; lanes 32..63: zero of row lane - 32
        const uint32_t so = gv ? (uint32_t)((lane & 31) * ng + (g * 128) / group) * 4 : kOutOfRange;
        const float sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, lane < 32 ? so : kOutOfRange, 0, 0));
        const float zv = SYM ? 0.0f
                             : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, lane >= 32 ? so : kOutOfRange, 0, 0));
        L.sz = lane < 32 ? sv : zv;
    };
    auto compute = [&](const GroupLoads &L) {
        // scales / zeros of rows 4 kq + v of each tile, via the wave's LDS slice
        sz_lds[wave][lane] = L.sz;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][4 * kq]);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][16 + 4 * kq]);
        f32x4 z0 = f32x4{0.f, 0.f, 0.f, 0.f}, z1 = z0;
        if (!SYM) {
            z0 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][32 + 4 * kq]);
            z1 = *reinterpret_cast<const f32x4 *>(&sz_lds[wave][48 + 4 * kq]);
        }
        // the next group's writes must not pass these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 d0 = f32x4{0.f, 0.f, 0.f, 0.f}, d1 = d0, xg = d0;
        const uint32_t w0[4] = {L.cw0.x, L.cw0.y, L.cw0.z, L.cw0.w};
        const uint32_t w1[4] = {L.cw1.x, L.cw1.y, L.cw1.z, L.cw1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, L.xv[j]);
            const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, unpack_natural(w0[j], magic));
            const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, unpack_natural(w1[j], magic));
            xg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bop, xg, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bop, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bop, d1, 0, 0, 0);
        }
        // lane holds D[row 4 kq + v][col l16]; X_g of column l16 in every v
        const float c = 128.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float c0 = SYM ? 136.0f : c + z0[v];
            const float c1 = SYM ? 136.0f : c + z1[v];
            acc0[v] = __builtin_fmaf(s0[v], __builtin_fmaf(-c0, xg[v], d0[v]), acc0[v]);
            acc1[v] = __builtin_fmaf(s1[v], __builtin_fmaf(-c1, xg[v], d1[v]), acc1[v]);
        }
    };

    if (g_begin < g_end) {
        // two groups per trip, both computed unconditionally: a conditional
        // exit between a load and its use would let the compiler sink the
        // prefetch to the use
        GroupLoads A, Bn;
        issue(g_begin, A);
        for (int g = g_begin; g < g_end; g += 2) {
            issue(g + 1, Bn);
            __builtin_amdgcn_sched_barrier(0);
            compute(A);
            issue(g + 2, A);
            __builtin_amdgcn_sched_barrier(0);
            compute(Bn);
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        red[wave][0][4 * kq + v][l16] = acc0[v];
        red[wave][1][4 * kq + v][l16] = acc1[v];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 2 * 256; e += blockDim.x) {
        const int t = e >> 8, rr = (e >> 4) & 15, col = e & 15;
        float v = 0.0f;
        for (int w = 0; w < nwaves; ++w) v += red[w][t][rr][col];
        const int row = row0 + t * 16 + rr;
        if (row < n && col < bsz) y[(int64_t)col * n + row] = v;
    }
}

// ---------------------------------------------------------------------------
// Ring kernel, batch 5..16 (v_mfma_f32_16x16x32_bf16, operands through LDS).
// A block's 4 waves share a tile of 16 weight rows and split k into
// 256-wide stages round-robin. Each wave streams its stages into a private
// LDS ring with buffer loads in the LDS-write form: the tile's codes (whole
// 128-byte lines of every row), XR (8 or 16) batch rows of activations (512
// bytes each; rows past the batch read zeros) and the two groups' scales and
// zeros of every row. Slots per wave: as many as fit in kRingWaveBytes
// (3 for XR = 16, 5 for XR = 8), so 1 or 3 stages stay in flight beyond the
// one being computed. It reads MFMA fragments from LDS:
// A = 16 rows x 32 k of codes (lane row l % 16, k quarter l / 16, natural
// unpack, one 16-byte read covers a group's four k-steps), B = 32 k x 16
// batch columns of activations. Per group the tile D_g and the activation
// sums X_g (an MFMA against a bf16 ones operand) give
// acc += s (D_g - (128 + z) X_g). The waves never wait for each other inside
// the loop (only for their own loads); they reduce through LDS at the end.
// LDS layout of a slot: codes [16 rows][128 B], 16-byte chunk c of row r
// stored at c ^ ((r >> 1) & 7); activations [XR rows][512 B], chunk c of row
// r at c ^ r (batch column b reads row b % XR; columns past the batch are
// never stored); scales, then zeros, [64] fp32 with entry 16 g + row for
// group g of the stage (entries 32..63 unused). With these the 16 rows
// (columns) of one fragment read fall in distinct banks.
// ---------------------------------------------------------------------------
constexpr int kRingStageK = 256;
constexpr int kRingWaveBytes = 33792;  // LDS ring of one wave
constexpr int kRingCodes = 16 * 128;
constexpr int kRingS = 256;            // scales, then zeros (symmetric leaves zeros unused)
constexpr int ring_slot(int xr) { return kRingCodes + xr * 512 + 2 * kRingS; }
constexpr int ring_slots(int xr) { return kRingWaveBytes / ring_slot(xr); }
constexpr int ring_loads(int xr, bool sym) { return 2 + xr / 2 + (sym ? 1 : 2); }  // LDS-write loads per stage
// vmcnt in the stage wait: (slots - 2) stages of younger loads, for
// XR = 16 / 8 and symmetric / asymmetric (literals: pasted into the asm)
#define LQ_GEMV_RING_VM_16S 11
#define LQ_GEMV_RING_VM_16A 12
#define LQ_GEMV_RING_VM_8S 21
#define LQ_GEMV_RING_VM_8A 24

#define LQ_GEMV_STR2(x) #x
#define LQ_GEMV_STR(x) LQ_GEMV_STR2(x)

template <int XR, bool SYM>
__global__ __launch_bounds__(256) void gemv_ring_kernel(const uint16_t *__restrict__ x, int bsz,
                                                         const uint8_t *__restrict__ codes,
                                                         const float *__restrict__ scales,
                                                         const float *__restrict__ zeros, int n, int k,
                                                         int group, float *__restrict__ y) {
    constexpr int kSlot = ring_slot(XR), kSlots = ring_slots(XR), kXP = XR / 2;
    static_assert(ring_loads(XR, SYM) * (kSlots - 2) ==
                      (XR == 16 ? (SYM ? LQ_GEMV_RING_VM_16S : LQ_GEMV_RING_VM_16A)
                                : (SYM ? LQ_GEMV_RING_VM_8S : LQ_GEMV_RING_VM_8A)),
                  "ring vmcnt");
    // one fixed-size array (a lambda capturing an array whose size depends on
    // a template parameter is dropped from the host compilation)
    // the only LDS array: with a second one declared the compiler waits for
    // all of a wave's LDS-write loads before every fragment read
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kRingWaveBytes];
    // after the loop each wave's partial sums [16][17] go to the start of its
    // own ring region
    auto red = [&](int w) { return reinterpret_cast<float (*)[17]>(ring + w * kRingWaveBytes); };
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    const int row0 = blockIdx.x * 16;
    const int ng = k / group;
    const uint32_t row_bytes = (uint32_t)k / 2;
    const int nst = (k + kRingStageK - 1) / kRingStageK;  // stages of this row range
    // descriptors: one per 16-row tile of codes; activations of the batch;
    // scales / zeros of the block's rows (rows past n read zeros)
    const int tile_rows = n - row0 < 16 ? n - row0 : 16;
    const auto rc = make_rsrc(codes + (int64_t)row0 * row_bytes, (uint32_t)tile_rows * row_bytes);
    const auto rx = make_rsrc(x, (uint32_t)bsz * (uint32_t)k * 2);
    const int rows_here = tile_rows;
    const auto rs = make_rsrc(scales + (int64_t)row0 * ng, (uint32_t)rows_here * ng * 4);
    const auto rz = make_rsrc(SYM ? scales : zeros + (int64_t)row0 * ng, SYM ? 0u : (uint32_t)rows_here * ng * 4);

    // per-lane source offsets of this wave's pieces (stage 0)
    // codes piece p: tile p / 2, rows 8 (p % 2) + l / 8, physical chunk l % 8
    // (fixed-size arrays: a lambda capturing an array whose size depends on a
    // template parameter is dropped from the host compilation)
    uint32_t c_off[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 8 * (p & 1) + (lane >> 3);
        c_off[p] = (uint32_t)r * row_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    // activation piece q: rows 2 q + l / 32, physical chunk l % 32
    uint32_t x_off[8];
#pragma unroll
    for (int q = 0; q < kXP; ++q) {
        const int xr = 2 * q + (lane >> 5);
        x_off[q] = (uint32_t)xr * (uint32_t)k * 2 + 16u * (uint32_t)((lane & 31) ^ xr);
    }
    // scales / zeros: lane l < 32 -> group-in-stage l / 16, row l % 16
    const int sz_grp = (lane >> 4) & 1;

    auto issue = [&](int st) {
        uint8_t *slot = ring + wave * kRingWaveBytes + (st % kSlots) * kSlot;
        const bool in = st < nst;  // later stages only keep the load count uniform
#pragma unroll
        for (int p = 0; p < 2; ++p)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (__attribute__((address_space(3))) void *)(slot + 1024 * p), 16,
                in ? c_off[p] + (uint32_t)st * 128 : kOutOfRange, 0, 0, kNonTemporal);
#pragma unroll
        for (int q = 0; q < kXP; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(slot + kRingCodes + 1024 * q), 16,
                in ? x_off[q] + (uint32_t)st * 512 : kOutOfRange, 0, 0, 0);
        // groups past k (a half last stage) read zeros: no contribution.
        // Group indices of the stage's two 128-wide groups: wave-uniform.
        const int gi0 = (st * kRingStageK) / group, gi1 = (st * kRingStageK + 128) / group;
        const bool gv = in && lane < 32 && (st * 2 + sz_grp) * 128 < k;
        const uint32_t gi = (uint32_t)(sz_grp ? gi1 : gi0);
        const uint32_t so = gv && l16 < rows_here ? (uint32_t)(l16 * ng) * 4 + gi * 4 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(slot + kRingCodes + XR * 512), 4, so, 0, 0, 0);
        if (!SYM)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rz, (__attribute__((address_space(3))) void *)(slot + kRingCodes + XR * 512 + kRingS), 4, so, 0, 0, 0);
    };

    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{kOnes, kOnes, kOnes, kOnes});
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment offsets within a slot
    int a_off[2];  // A of row l16, group h: logical chunk 4 h + kq
#pragma unroll
    for (int h = 0; h < 2; ++h) a_off[h] = l16 * 128 + 16 * ((4 * h + kq) ^ ((l16 >> 1) & 7));
    int b_off[2][4];  // B of column l16 (row l16 % XR), group h, step j: logical chunk 16 h + 4 kq + j
    const int xrow = l16 % XR;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) b_off[h][j] = kRingCodes + xrow * 512 + 16 * ((16 * h + 4 * kq + j) ^ xrow);

    const int my_stages = wave < nst ? (nst - wave + 3) / 4 : 0;
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i) issue(wave + 4 * i);
    for (int i = 0; i < my_stages; ++i) {
        // this wave's loads of stage i are done once at most (slots - 2)
        // stages of younger loads are pending (the compiler does not track
        // LDS-write loads). The slot the issue below refills was last read
        // by stage i - 1, whose fragments this wave has consumed.
        if (XR == 16 && SYM)
            asm volatile("s_waitcnt vmcnt(" LQ_GEMV_STR(LQ_GEMV_RING_VM_16S) ")" ::: "memory");
        else if (XR == 16)
            asm volatile("s_waitcnt vmcnt(" LQ_GEMV_STR(LQ_GEMV_RING_VM_16A) ")" ::: "memory");
        else if (SYM)
            asm volatile("s_waitcnt vmcnt(" LQ_GEMV_STR(LQ_GEMV_RING_VM_8S) ")" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(" LQ_GEMV_STR(LQ_GEMV_RING_VM_8A) ")" ::: "memory");
        issue(wave + 4 * (i + kSlots - 1));
        const uint8_t *slot = ring + wave * kRingWaveBytes + ((wave + 4 * i) % kSlots) * kSlot;
        const float *sz = reinterpret_cast<const float *>(slot + kRingCodes + XR * 512);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8_t bop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bop[j] = *reinterpret_cast<const bf16x8_t *>(slot + b_off[h][j]);
            f32x4 xg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) xg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bop[j], xg, 0, 0, 0);
            const u32x4 cw = *reinterpret_cast<const u32x4 *>(slot + a_off[h]);
            const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
            f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, unpack_natural(w[j], magic)),
                                                            bop[j], d, 0, 0, 0);
            // rows 4 kq + v of the tile: scales at [16 h + row], zeros 64 entries later
            const f32x4 sv = *reinterpret_cast<const f32x4 *>(&sz[h * 16 + 4 * kq]);
            f32x4 zv = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!SYM) zv = *reinterpret_cast<const f32x4 *>(&sz[64 + h * 16 + 4 * kq]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float c = SYM ? 136.0f : 128.0f + zv[v];
                acc[v] = __builtin_fmaf(sv[v], __builtin_fmaf(-c, xg[v], d[v]), acc[v]);
            }
        }
    }
    // drain the trailing (out-of-range) loads before the LDS is reused; the
    // builtin also tells the compiler nothing is pending
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (gfx9 layout)
#pragma unroll
    for (int v = 0; v < 4; ++v) red(wave)[4 * kq + v][l16] = acc[v];
    __syncthreads();
    {
        const int rr = threadIdx.x >> 4, col = threadIdx.x & 15;
        const float v = red(0)[rr][col] + red(1)[rr][col] + red(2)[rr][col] + red(3)[rr][col];
        const int row = row0 + rr;
        if (row < n && col < bsz) y[(int64_t)col * n + row] = v;
    }
}

template <int B, int RW, bool SYM, int WPB = 4>
static hipError_t launch_valu_rw(const WoArgs &a, hipStream_t st, int ks_count) {
    // staged scales need whole 4-group runs per row: k a multiple of 512
    const bool g128 = a.group == 128 && a.k % 512 == 0;
    const int rows_per_block = (WPB / ks_count) * RW;
    const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
    if (g128)
        hipLaunchKernelGGL((gemv_valu_kernel<B, RW, SYM, true, WPB>), dim3((uint32_t)blocks), dim3(WPB * 64), 0, st,
                           a.x, a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, ks_count, a.y);
    else
        hipLaunchKernelGGL((gemv_valu_kernel<B, RW, SYM, false, WPB>), dim3((uint32_t)blocks), dim3(WPB * 64), 0,
                           st, a.x, a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, ks_count, a.y);
    return hipGetLastError();
}

// Launch shape (measured on MI355X): the block's four waves split k four
// ways when a row has 4..7 chunks, two ways when it has 2..3 or 8 and more
// (then each wave walks several chunks), not at all for one chunk. A wave
// takes 8 rows, except where 4 rows measured faster: with one chunk, below
// 512 blocks of 8 rows; with the four-way split, at up to 512 blocks
// (4096 x 11008: 7.7 against 8.3 us). With the two-way split 8 rows win
// also on 256 blocks (4096 x 4096: 4.2 against 4.4 us). At batch 1 with 5..7
// chunks, blocks of 8 waves split k eight ways, so that no wave walks a
// second chunk after its first (4 rows a wave; 4096 x 11008: 7.0 against
// 7.85 us; with 4 or 8 chunks, and 14, the four-wave shapes are as fast).
template <int B, bool SYM>
static hipError_t launch_valu(const WoArgs &a, hipStream_t st) {
    const int nchunks = (int)((a.k + kChunk - 1) / kChunk);
    if (B == 1 && nchunks >= 5 && nchunks <= 7) return launch_valu_rw<B, 4, SYM, 8>(a, st, 8);
    const int ks = nchunks >= 8 ? 2 : nchunks >= 4 ? 4 : nchunks >= 2 ? 2 : 1;
    const int64_t blocks8 = (a.n + (4 / ks) * 8 - 1) / ((4 / ks) * 8);
    const bool rw8 = ks == 2 ? true : ks == 4 ? blocks8 > 512 : blocks8 >= 512;
    return rw8 ? launch_valu_rw<B, 8, SYM>(a, st, ks) : launch_valu_rw<B, 4, SYM>(a, st, ks);
}

// Waves per block: enough to put about 2048 waves on the chip (8 per CU),
// 4 to 16, and no more than there are groups; then the runs are balanced.
template <bool SYM>
static hipError_t launch_mfma(const WoArgs &a, hipStream_t st) {
    const int64_t blocks = (a.n + kMfmaRows - 1) / kMfmaRows;
    const int ng128 = (int)(a.k / 128);
    int wpb = 4;
    while (wpb < 16 && blocks * wpb < 2048) wpb *= 2;
    wpb = wpb < ng128 ? wpb : ng128;
    const int gpw = (ng128 + wpb - 1) / wpb;
    wpb = (ng128 + gpw - 1) / gpw;
    hipLaunchKernelGGL((gemv_mfma_kernel<SYM>), dim3((uint32_t)blocks), dim3(64 * wpb), 0, st, a.x, (int)a.m,
                       a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, gpw, a.y);
    return hipGetLastError();
}

// Batch 4..16 on large matrices: the shared-stage kernel of gemv_shared.hip.
static hipError_t launch_shared(const WoArgs &a, hipStream_t st) {
    const SharedGemvArgs sa{a.x, a.m, a.codes, a.scales, a.zeros, a.n, a.k, a.symmetric, a.group, a.y};
    return launch_shared_gemv(WeightFormat::kInt4, sa, st);
}

// Batch 5..16 elsewhere (measured on MI355X): the LDS-ring kernel while
// there are few 16-row tiles (n <= 12288: up to 768 blocks) and its
// activation descriptor (batch x k x 2 bytes) fits 32 bits; the
// register-streaming MFMA kernel for taller matrices.
template <bool SYM>
static hipError_t launch_batch(const WoArgs &a, hipStream_t st) {
    if (shared_gemv_pays(WeightFormat::kInt4, a.m, a.n, a.k)) return launch_shared(a, st);
    if (a.n <= 12288 && a.m * a.k * 2 < (int64_t(1) << 32)) {
        if (a.m <= 8)
            hipLaunchKernelGGL((gemv_ring_kernel<8, SYM>), dim3((uint32_t)((a.n + 15) / 16)), dim3(256), 0, st, a.x,
                               (int)a.m, a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, a.y);
        else
            hipLaunchKernelGGL((gemv_ring_kernel<16, SYM>), dim3((uint32_t)((a.n + 15) / 16)), dim3(256), 0, st, a.x,
                               (int)a.m, a.codes, a.scales, a.zeros, (int)a.n, (int)a.k, (int)a.group, a.y);
        return hipGetLastError();
    }
    return launch_mfma<SYM>(a, st);
}

template <bool SYM>
static hipError_t launch_gemv_s(const WoArgs &a, hipStream_t st) {
    switch (a.m) {
        case 1: return launch_valu<1, SYM>(a, st);
        case 2: return launch_valu<2, SYM>(a, st);
        case 3: return launch_valu<3, SYM>(a, st);
        case 4:
            return shared_gemv_pays(WeightFormat::kInt4, a.m, a.n, a.k) ? launch_shared(a, st)
                                                                        : launch_valu<4, SYM>(a, st);
        default: return launch_batch<SYM>(a, st);
    }
}

hipError_t launch_w4a16_gemv(const WoArgs &a, hipStream_t st) {
    if (a.m < 1 || a.m > 16) return hipErrorInvalidValue;
    return a.symmetric ? launch_gemv_s<true>(a, st) : launch_gemv_s<false>(a, st);
}

}  // namespace lq
