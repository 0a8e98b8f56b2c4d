// quantize.hip -- group-wise RTN quantize/pack and dequantize for gfx950.
//
// Definition: "3.6 Quantization" (LLM learning path), section "Symmetric and
// asymmetric quantization" and its code block (1e-8 floor on range/absmax,
// torch.round = round half to even); "Quantization: trading precision for
// performance" (mokono.cn) 2.3: q = round(x / s) + z, x_hat = (q - z) s.
//
// Both passes stream HBM once. Every scale, zero and code is produced with
// the same fp32 operations, in the same order, as the IEEE definition:
// correctly rounded division (the HIP default), rintf = round half to even,
// no FMA contraction (the library is built with -ffp-contract=off).
#include "common.hpp"
#include "launch.hpp"

namespace lq {

// Statistics of one group, reduced over a team of lanes, then s and z.
template <bool SYM>
struct GroupStats {
    float a;   // symmetric: running max |x|
    float mn;  // asymmetric: running min
    float mx;  // asymmetric: running max
    LQ_DEVICE void init() {
        a = 0.0f;
        mn = __builtin_inff();
        mx = -__builtin_inff();
    }
    LQ_DEVICE void add(float v) {
        if (SYM) {
            a = fmaxf(a, fabsf(v));
        } else {
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
    }
};

template <int BITS, bool SYM>
LQ_DEVICE void scale_zero(float a, float mn, float mx, float &s, float &z) {
    if (SYM) {
        const float qmax = (float)((1 << (BITS - 1)) - 1);
        float am = a < kFloor ? kFloor : a;
        s = am / qmax;
        z = 0.0f;
    } else {
        const float levels = (float)((1 << BITS) - 1);
        float range = mx - mn;
        range = range < kFloor ? kFloor : range;
        s = range / levels;
        z = rintf(-mn / s) + 0.0f;  // "+ 0.0f": -0 -> +0
    }
}

// Integer code of one element from its quotient x / s (before the INT4
// symmetric +8 offset).
template <int BITS, bool SYM>
LQ_DEVICE int code_of_quotient(float qd, float z) {
    if (SYM) {
        const float qmax = (float)((1 << (BITS - 1)) - 1);
        return (int)clamp_code(rintf(qd), -qmax, qmax);
    } else {
        const float levels = (float)((1 << BITS) - 1);
        const float r = rintf(qd) + z;  // round first, then add z
        return (int)clamp_code(r, 0.0f, levels);
    }
}

// Quotients through div_rn (common.hpp; Markstein's division): it equals the
// IEEE quotient while every intermediate is normal and finite. The fast
// path of a group (magnitudes at most 2^59) uses it for
//  * the scale, range or absmax (at least 1e-8) over the level count: all
//    intermediates are at least about 1e-8 * 2^-24, hence normal;
//  * quotients that are then rounded to an integer, with divisor s in
//    [1e-8 / 255, 2^60 / 7]: a quotient of magnitude 1/2 or more has
//    |a| >= s / 2, so its residual is normal too; smaller ones round to
//    zero under either path.

// Fast path of a group: every magnitude at most 2^59. Then s lies in
// [1e-8 / 255, 2^60 / 7] (range or absmax floored at 1e-8), every quotient
// x / s, -mn / s and range / levels meets div_rn's conditions, and nothing
// is infinite or NaN, so the clamp may use v_med3.
constexpr float kFastMax = 5.76460752303423488e+17f;  // 2^59
LQ_DEVICE bool fast_group(float amax) { return amax <= kFastMax; }

// Scale, zero and reciprocal scale on the fast path: the same values as
// scale_zero (divisions by the level count through div_rn with the constant
// RN(1 / levels)).
template <int BITS, bool SYM>
LQ_DEVICE void scale_zero_fast(float a, float mn, float mx, float &s, float &z, float &y) {
    if (SYM) {
        constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
        const float am = a < kFloor ? kFloor : a;
        s = div_rn(am, qmax, 1.0f / qmax);
        y = 1.0f / s;
        z = 0.0f;
    } else {
        constexpr float levels = (float)((1 << BITS) - 1);
        float range = mx - mn;
        range = range < kFloor ? kFloor : range;
        s = div_rn(range, levels, 1.0f / levels);
        y = 1.0f / s;
        z = rintf(div_rn(-mn, s, y)) + 0.0f;  // "+ 0.0f": -0 -> +0
    }
}

LQ_DEVICE void unpack8(const u32x4 v, float x[8]) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// NT: streaming (nontemporal) load for data read exactly once.
template <bool CS, bool NT>
LQ_DEVICE void load8(const uint16_t *__restrict__ w, const float *__restrict__ cs, int64_t elem,
                     int64_t col, float x[8]) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(w + elem);
    const u32x4 v = NT ? __builtin_nontemporal_load(p) : *p;
    unpack8(v, x);
    if (CS) {
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cs + col);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cs + col + 4);
        x[0] = x[0] * c0.x; x[1] = x[1] * c0.y; x[2] = x[2] * c0.z; x[3] = x[3] * c0.w;
        x[4] = x[4] * c1.x; x[5] = x[5] * c1.y; x[6] = x[6] * c1.z; x[7] = x[7] * c1.w;
    }
}

// Codes of 8 consecutive elements -> packed storage.
template <int BITS, bool SYM>
LQ_DEVICE void store8(uint8_t *__restrict__ codes, int64_t elem, const int q[8]) {
    if (BITS == 4) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= (uint32_t)((SYM ? q[i] + 8 : q[i]) & 0xF) << (4 * i);
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes + elem / 2));
    } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (uint32_t)(q[i] & 0xFF) << (8 * i);
            hi |= (uint32_t)(q[i + 4] & 0xFF) << (8 * i);
        }
        u32x2 v;
        v.x = lo;
        v.y = hi;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(codes + elem));
    }
}

// Fast path (finite values, so v_med3 is the clamp): the stored code of a
// quotient as an exact small integer in a float, offset for storage -- INT4 asymmetric c, INT4 symmetric c + 8,
// INT8 asymmetric c, INT8 symmetric c + 128 (the byte is flipped back to
// two's complement by the packing) -- so that two codes combine with one FMA
// and a byte is placed with one v_cvt_pk_u8_f32 (exact for integers in
// [0, 255]). Measured on MI355X: 8-10 % less time for the G = 128 kernel
// than converting each code to an integer and shifting it into place.
template <int BITS, bool SYM>
LQ_DEVICE float stored_code_fast(float qd, float z) {
    if (SYM) {
        constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
        constexpr float off = BITS == 4 ? 8.0f : 128.0f;
        return __builtin_amdgcn_fmed3f(rintf(qd) + off, off - qmax, off + qmax);  // rint(qd) is exact + off
    } else {
        constexpr float levels = (float)((1 << BITS) - 1);
        return __builtin_amdgcn_fmed3f(rintf(qd) + z, 0.0f, levels);
    }
}

// Eight INT4 stored codes (from stored_code_fast) -> one word, element i at
// bits 4i .. 4i + 3.
LQ_DEVICE uint32_t pack8_int4(const float c[8]) {
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c[2 * p + 1], 16.0f, c[2 * p]), p, word);
    return word;
}

// Stored codes of 8 consecutive elements (from stored_code_fast) -> packed.
template <int BITS, bool SYM>
LQ_DEVICE void store8_fast(uint8_t *__restrict__ codes, int64_t elem, const float c[8]) {
    if (BITS == 4) {
        uint32_t word = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c[2 * p + 1], 16.0f, c[2 * p]), p, word);
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes + elem / 2));
    } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            lo = __builtin_amdgcn_cvt_pk_u8_f32(c[p], p, lo);
            hi = __builtin_amdgcn_cvt_pk_u8_f32(c[p + 4], p, hi);
        }
        if (SYM) {
            lo ^= 0x80808080u;
            hi ^= 0x80808080u;
        }
        u32x2 v;
        v.x = lo;
        v.y = hi;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(codes + elem));
    }
}

// Max / min over each aligned team of TS (16 or 8) lanes, result in every
// lane: the DPP partners l ^ 15 (16-lane teams only), l ^ 7, l ^ 2, l ^ 1
// together reach every lane of the team.
template <int TS>
LQ_DEVICE float team_dpp_max(float v) {
    static_assert(TS == 16 || TS == 8, "teams of 16 or 8 lanes");
    if (TS == 16) v = fmaxf(v, dpp_move<kDppMirror>(v));
    v = fmaxf(v, dpp_move<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_move<kDppXor2>(v));
    return fmaxf(v, dpp_move<kDppXor1>(v));
}
template <int TS>
LQ_DEVICE float team_dpp_min(float v) {
    static_assert(TS == 16 || TS == 8, "teams of 16 or 8 lanes");
    if (TS == 16) v = fminf(v, dpp_move<kDppMirror>(v));
    v = fminf(v, dpp_move<kDppHalfMirror>(v));
    v = fminf(v, dpp_move<kDppXor2>(v));
    return fminf(v, dpp_move<kDppXor1>(v));
}

// Groups of G = 8 TS M elements: a team of TS lanes (16 or 8) owns a group,
// 8 elements (16 bytes of bf16) per lane in each of its M chunks of 8 TS
// elements, and each team takes GPT groups. A block's (256 / TS) GPT groups
// are contiguous; load (i, c) covers chunk c of one group per team, 16 TS
// contiguous bytes (whole 128-byte lines); all GPT M loads are issued before
// any group is computed. Groups tile the rows contiguously (G divides k), so
// group index g covers elements [G g, G g + G) of the flattened matrix and
// its scale sits at scales[g].
template <int BITS, bool SYM, bool CS, int TS, int M, int GPT>
__global__ __launch_bounds__(256) void quant_team_kernel(const uint16_t *__restrict__ w,
                                                          int64_t ngroups, int64_t k,
                                                          const float *__restrict__ cs,
                                                          uint8_t *__restrict__ codes,
                                                          float *__restrict__ scales,
                                                          float *__restrict__ zeros, int64_t cs_stride,
                                                          int64_t code_stride, int64_t meta_stride) {
    // batch member blockIdx.y (a batch of column scalings of the same W)
    if (CS) cs += blockIdx.y * cs_stride;
    codes += blockIdx.y * code_stride;
    scales += blockIdx.y * meta_stride;
    if (!SYM) zeros += blockIdx.y * meta_stride;
    constexpr int kTeams = 256 / TS;
    constexpr int kChunk = 8 * TS;
    constexpr int G = kChunk * M;
    // INT4 with 128-element groups on 8-lane teams: a group's 64 code bytes
    // leave in one store per team (whole lines with the neighbouring team)
    // instead of two half-filled ones
    constexpr bool kWholeLines = BITS == 4 && TS == 8 && M == 2;
    const int team = threadIdx.x / TS;
    const int l = threadIdx.x % TS;
    const int64_t g0 = (int64_t)blockIdx.x * (kTeams * GPT) + team;
    float x[GPT][M][8];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int64_t g = g0 + kTeams * i;
        if (g < ngroups) {  // team-uniform
#pragma unroll
            for (int c = 0; c < M; ++c) {
                const int64_t elem = g * G + kChunk * c + l * 8;
                load8<CS, true>(w, cs, elem, CS ? elem % k : 0, x[i][c]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int64_t g = g0 + kTeams * i;
        if (g >= ngroups) break;  // team-uniform; later groups are past the end too
        GroupStats<SYM> st;
        st.init();
#pragma unroll
        for (int c = 0; c < M; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) st.add(x[i][c][j]);
        float a = 0.f, mn = 0.f, mx = 0.f;
        if (SYM) {
            a = team_dpp_max<TS>(st.a);
        } else {
            mn = team_dpp_min<TS>(st.mn);
            mx = team_dpp_max<TS>(st.mx);
        }
        float s, z;
        // the 16-lane team takes one branch: it shares the extremes
        if (fast_group(SYM ? a : fmaxf(-mn, mx))) {
            float y;
            scale_zero_fast<BITS, SYM>(a, mn, mx, s, z, y);
            if constexpr (kWholeLines) {
                // the two code words of the lane, then the team's 64 bytes in
                // one store: lane l takes elements 16 l .. 16 l + 15, i.e. the
                // words of lanes 2 l and 2 l + 1 of chunk l / 4
                uint32_t word[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float cf[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) cf[j] = stored_code_fast<BITS, SYM>(div_rn(x[i][c][j], s, y), z);
                    word[c] = pack8_int4(cf);
                }
                const int s0 = (2 * l) & 7;
                const int a0 = __shfl((int)word[0], s0, 8), b0 = __shfl((int)word[1], s0, 8);
                const int a1 = __shfl((int)word[0], s0 + 1, 8), b1 = __shfl((int)word[1], s0 + 1, 8);
                const u32x2 v{(uint32_t)(l < 4 ? a0 : b0), (uint32_t)(l < 4 ? a1 : b1)};
                __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(codes + (g * G) / 2 + 8 * l));
            } else {
#pragma unroll
                for (int c = 0; c < M; ++c) {
                    float cf[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) cf[j] = stored_code_fast<BITS, SYM>(div_rn(x[i][c][j], s, y), z);
                    store8_fast<BITS, SYM>(codes, g * G + kChunk * c + l * 8, cf);
                }
            }
        } else {
            scale_zero<BITS, SYM>(a, mn, mx, s, z);
#pragma unroll
            for (int c = 0; c < M; ++c) {
                int q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = code_of_quotient<BITS, SYM>(x[i][c][j] / s, z);
                store8<BITS, SYM>(codes, g * G + kChunk * c + l * 8, q);
            }
        }
        if (l == 0) {
            scales[g] = s;
            if (!SYM) zeros[g] = z;
        }
    }
}

// Groups above 1024 elements (per-channel rows of k > 1024 included): one block of
// TPB lanes per group, read in chunks of kBigLoads * TPB * 8 elements (each
// lane's kBigLoads 16-byte loads issued before any arithmetic). Statistics
// run over every chunk, then codes are formed from the chunk still in
// registers and from re-reads of the others, so a group of up to one chunk
// is read from memory once: 8192 elements with 256 lanes, 32768 with 1024.
// Measured on MI355X, INT8 per channel with column scales, weights cold in
// HBM: 8192 x 8192 in 42 us, 28672 x 8192 in 143 us, where one dependent
// load at a time per lane took 63 and 202 us.
constexpr int kBigLoads = 4;

// Elements c0 + 8 t + 8 TPB i .. + 7 (i < kBigLoads) of the group at `base`,
// times their column scales; lanes past the group read nothing.
template <int TPB, bool CS, bool NT>
LQ_DEVICE void load_chunk(const uint16_t *__restrict__ w, const float *__restrict__ cs, int64_t base,
                          int64_t group, int64_t k, int64_t c0, int t, float x[kBigLoads][8]) {
    u32x4 v[kBigLoads];
    f32x4 c[kBigLoads][2];
#pragma unroll
    for (int i = 0; i < kBigLoads; ++i) {
        const int64_t e = c0 + t * 8 + 8 * TPB * i;
        const bool in = e < group;
        const u32x4 *p = reinterpret_cast<const u32x4 *>(w + base + e);
        v[i] = !in ? u32x4{0u, 0u, 0u, 0u} : NT ? __builtin_nontemporal_load(p) : *p;
        if (CS) {
            const int64_t col = in ? (base + e) % k : 0;
            c[i][0] = *reinterpret_cast<const f32x4 *>(cs + col);
            c[i][1] = *reinterpret_cast<const f32x4 *>(cs + col + 4);
        }
    }
#pragma unroll
    for (int i = 0; i < kBigLoads; ++i) {
        unpack8(v[i], x[i]);
        if (CS) {
            x[i][0] *= c[i][0].x; x[i][1] *= c[i][0].y; x[i][2] *= c[i][0].z; x[i][3] *= c[i][0].w;
            x[i][4] *= c[i][1].x; x[i][5] *= c[i][1].y; x[i][6] *= c[i][1].z; x[i][7] *= c[i][1].w;
        }
    }
}

// ONE: the group fits one chunk (read once, streaming).
template <int BITS, bool SYM, bool CS, bool ONE, int TPB>
__global__ __launch_bounds__(TPB) void quant_big_kernel(const uint16_t *__restrict__ w, int64_t group,
                                                         int64_t k, const float *__restrict__ cs,
                                                         uint8_t *__restrict__ codes,
                                                         float *__restrict__ scales,
                                                         float *__restrict__ zeros) {
    constexpr int kWaves = TPB / 64;
    constexpr int64_t kChunk = (int64_t)kBigLoads * TPB * 8;
    __shared__ float red[3][kWaves];
    const int64_t g = blockIdx.x;
    const int64_t base = g * group;
    const int t = threadIdx.x;
    const int64_t nch = ONE ? 1 : (group + kChunk - 1) / kChunk;
    GroupStats<SYM> st;
    st.init();
    float x[kBigLoads][8];
    for (int64_t ch = 0; ch < nch; ++ch) {
        load_chunk<TPB, CS, ONE>(w, cs, base, group, k, ch * kChunk, t, x);
#pragma unroll
        for (int i = 0; i < kBigLoads; ++i)
            if (ch * kChunk + t * 8 + 8 * TPB * i < group) {
#pragma unroll
                for (int j = 0; j < 8; ++j) st.add(x[i][j]);
            }
    }
    float a = 0.f, mn = 0.f, mx = 0.f;
    if (SYM) {
        a = team_max<64>(st.a);
    } else {
        mn = team_min<64>(st.mn);
        mx = team_max<64>(st.mx);
    }
    const int wave = t >> 6;
    if ((t & 63) == 0) {
        red[0][wave] = a;
        red[1][wave] = mn;
        red[2][wave] = mx;
    }
    __syncthreads();
    a = red[0][0];
    mn = red[1][0];
    mx = red[2][0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) {
        a = fmaxf(a, red[0][i]);
        mn = fminf(mn, red[1][i]);
        mx = fmaxf(mx, red[2][i]);
    }
    float s, z, y = 0.0f;
    const bool fast = fast_group(SYM ? a : fmaxf(-mn, mx));  // block-uniform
    if (fast)
        scale_zero_fast<BITS, SYM>(a, mn, mx, s, z, y);
    else
        scale_zero<BITS, SYM>(a, mn, mx, s, z);
    // the last chunk is still in x; the others are read again
    for (int64_t ch = nch - 1; ch >= 0; --ch) {
        if (ch != nch - 1) load_chunk<TPB, CS, false>(w, cs, base, group, k, ch * kChunk, t, x);
#pragma unroll
        for (int i = 0; i < kBigLoads; ++i) {
            const int64_t e = ch * kChunk + t * 8 + 8 * TPB * i;
            if (e >= group) continue;
            if (fast) {
                float c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = stored_code_fast<BITS, SYM>(div_rn(x[i][j], s, y), z);
                store8_fast<BITS, SYM>(codes, base + e, c);
            } else {
                int q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = code_of_quotient<BITS, SYM>(x[i][j] / s, z);
                store8<BITS, SYM>(codes, base + e, q);
            }
        }
    }
    if (t == 0) {
        scales[g] = s;
        if (!SYM) zeros[g] = z;
    }
}

// Per-channel rows with column scales (group == k, 1024 < k <= 8192): a
// block of 256 lanes takes R consecutive rows, which share their columns, so
// each lane loads the column scales of its elements once for R rows (they
// cost two 16-byte loads per 16 bytes of weights). The rows are held in
// registers, as in quant_big_kernel. Measured on MI355X, INT8 of W * s with
// W cold in HBM (one row per block -> two): 8192 x 8192 42.5 -> 39.6 us,
// 28672 x 8192 140 -> 126 us (the same rows without column scales: 35 us
// on 8192 x 8192); k = 4224 and 2048 were 10 % slower with two rows (half
// the blocks, fewer loads a lane), four rows were slower everywhere, so
// two rows are taken from k = 6144.
template <int BITS, bool SYM, int R>
__global__ __launch_bounds__(256) void quant_rows_cs_kernel(const uint16_t *__restrict__ w, int64_t nrows,
                                                             int64_t k, const float *__restrict__ cs,
                                                             uint8_t *__restrict__ codes,
                                                             float *__restrict__ scales,
                                                             float *__restrict__ zeros) {
    __shared__ float red[3][R][4];
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int t = threadIdx.x;
    float x[R][kBigLoads][8];
    {
        u32x4 v[R][kBigLoads];
        f32x4 c[kBigLoads][2];
#pragma unroll
        for (int i = 0; i < kBigLoads; ++i) {
            const int64_t e = t * 8 + 2048 * i;
            const bool in = e < k;
#pragma unroll
            for (int r = 0; r < R; ++r)
                v[r][i] = in && r0 + r < nrows
                              ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w + (r0 + r) * k + e))
                              : u32x4{0u, 0u, 0u, 0u};
            c[i][0] = *reinterpret_cast<const f32x4 *>(cs + (in ? e : 0));
            c[i][1] = *reinterpret_cast<const f32x4 *>(cs + (in ? e : 0) + 4);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < kBigLoads; ++i) {
                unpack8(v[r][i], x[r][i]);
                x[r][i][0] *= c[i][0].x; x[r][i][1] *= c[i][0].y; x[r][i][2] *= c[i][0].z; x[r][i][3] *= c[i][0].w;
                x[r][i][4] *= c[i][1].x; x[r][i][5] *= c[i][1].y; x[r][i][6] *= c[i][1].z; x[r][i][7] *= c[i][1].w;
            }
    }
    const int wave = t >> 6;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        GroupStats<SYM> st;
        st.init();
#pragma unroll
        for (int i = 0; i < kBigLoads; ++i)
            if (t * 8 + 2048 * i < k) {
#pragma unroll
                for (int j = 0; j < 8; ++j) st.add(x[r][i][j]);
            }
        float a = 0.f, mn = 0.f, mx = 0.f;
        if (SYM) {
            a = team_max<64>(st.a);
        } else {
            mn = team_min<64>(st.mn);
            mx = team_max<64>(st.mx);
        }
        if ((t & 63) == 0) {
            red[0][r][wave] = a;
            red[1][r][wave] = mn;
            red[2][r][wave] = mx;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = r0 + r;
        if (row >= nrows) break;  // block-uniform
        const float a = fmaxf(fmaxf(red[0][r][0], red[0][r][1]), fmaxf(red[0][r][2], red[0][r][3]));
        const float mn = fminf(fminf(red[1][r][0], red[1][r][1]), fminf(red[1][r][2], red[1][r][3]));
        const float mx = fmaxf(fmaxf(red[2][r][0], red[2][r][1]), fmaxf(red[2][r][2], red[2][r][3]));
        float s, z, y = 0.0f;
        const bool fast = fast_group(SYM ? a : fmaxf(-mn, mx));  // block-uniform
        if (fast)
            scale_zero_fast<BITS, SYM>(a, mn, mx, s, z, y);
        else
            scale_zero<BITS, SYM>(a, mn, mx, s, z);
#pragma unroll
        for (int i = 0; i < kBigLoads; ++i) {
            const int64_t e = t * 8 + 2048 * i;
            if (e >= k) continue;
            if (fast) {
                float c8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) c8[j] = stored_code_fast<BITS, SYM>(div_rn(x[r][i][j], s, y), z);
                store8_fast<BITS, SYM>(codes, row * k + e, c8);
            } else {
                int q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = code_of_quotient<BITS, SYM>(x[r][i][j] / s, z);
                store8<BITS, SYM>(codes, row * k + e, q);
            }
        }
        if (t == 0) {
            scales[row] = s;
            if (!SYM) zeros[row] = z;
        }
    }
}

// x_hat = (q - z) * s. A wave takes 512 consecutive elements and lane l the
// elements 4 l .. 4 l + 3 and 256 + 4 l .. + 3 of them, so each of its two
// 16-byte stores covers 1 KB of contiguous output (the output is 7 of every
// 8 bytes moved for INT4).
template <int BITS, bool SYM>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                       const float *__restrict__ scales,
                                                       const float *__restrict__ zeros,
                                                       int64_t total, int64_t group,
                                                       float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 512;
    // both halves' code, scale and zero loads first (a lane past the end
    // reads element 0 and stores nothing): 58.1 -> 55.6 us on 8192 x 8192
    uint32_t v[2];
    float s[2], z[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t elem = base + 256 * h + 4 * lane;  // total is a multiple of 128
        const int64_t e = elem < total ? elem : 0;
        v[h] = BITS == 4 ? (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(codes + e / 2))
                         : __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + e));
        const int64_t g = e / group;  // groups tile the flattened matrix
        s[h] = scales[g];
        z[h] = SYM ? 0.0f : zeros[g];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t elem = base + 256 * h + 4 * lane;
        if (elem >= total) continue;
        int q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (BITS == 4) {
                const int u = (int)((v[h] >> (4 * j)) & 0xF);
                q[j] = SYM ? u - 8 : u;
            } else {
                const uint32_t b = (v[h] >> (8 * j)) & 0xFF;
                q[j] = SYM ? (int)(int8_t)b : (int)b;
            }
        }
        // plain stores: the non-temporal hint measured 3-5 % slower here
        // (8192 x 8192 INT4 -> fp32, 55.5-58.3 against 52.9-55.1 us)
        *reinterpret_cast<f32x4 *>(out + elem) = f32x4{((float)q[0] - z[h]) * s[h], ((float)q[1] - z[h]) * s[h],
                                                       ((float)q[2] - z[h]) * s[h], ((float)q[3] - z[h]) * s[h]};
    }
}

// Team shapes (measured on MI355X, INT4 asymmetric, weights cold in HBM):
// G = 128 on 8-lane teams with two 64-element chunks per lane and two groups
// per team; 57344 x 8192 in 209-235 us against 243-305 us on 16-lane teams
// (the per-group extremes, scale and zero are formed by every lane of a
// team, so fewer lanes per group do less of that work) and 345 us on 4-lane
// teams (each load then covers parts of cache lines). G = 256 and 512 stay on
// 16-lane teams (two or four chunks per lane): 8-lane teams were 20-40 %
// slower there. G = 256: 203 us on the same matrix.
template <int BITS, bool SYM, bool CS, int TS, int M, int GPT>
static hipError_t launch_team(const QuantArgs &a, int64_t ngroups, hipStream_t st) {
    constexpr int64_t per_block = 256 / TS * GPT;
    const int64_t blocks = (ngroups + per_block - 1) / per_block;
    hipLaunchKernelGGL((quant_team_kernel<BITS, SYM, CS, TS, M, GPT>), dim3((uint32_t)blocks, (uint32_t)a.batch),
                       dim3(256), 0, st, a.w, ngroups, a.k, a.col_scale, a.codes, a.scales, a.zeros, a.cs_stride,
                       a.code_stride, a.meta_stride);
    return hipGetLastError();
}

template <int BITS, bool SYM, bool CS>
static hipError_t launch_quant_t(const QuantArgs &a, hipStream_t st) {
    const int64_t ngroups = a.n * (a.k / a.group);
    const bool team = a.group % 128 == 0 && a.group <= 128 * 8;
    if (a.batch > 1 && !team) {  // the other kernels take one product per launch
        for (int p = 0; p < a.batch; ++p) {
            QuantArgs one = a;
            one.batch = 1;
            one.col_scale = a.col_scale ? a.col_scale + p * a.cs_stride : nullptr;
            one.codes = a.codes + p * a.code_stride;
            one.scales = a.scales + p * a.meta_stride;
            one.zeros = a.zeros ? a.zeros + p * a.meta_stride : nullptr;
            const hipError_t e = launch_quant_t<BITS, SYM, CS>(one, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (team) {
        switch (a.group / 128) {
            case 1: return launch_team<BITS, SYM, CS, 8, 2, 2>(a, ngroups, st);
            case 2: return launch_team<BITS, SYM, CS, 16, 2, 2>(a, ngroups, st);
            case 3: return launch_team<BITS, SYM, CS, 16, 3, 1>(a, ngroups, st);
            case 4: return launch_team<BITS, SYM, CS, 16, 4, 1>(a, ngroups, st);
            case 5: return launch_team<BITS, SYM, CS, 16, 5, 1>(a, ngroups, st);
            case 6: return launch_team<BITS, SYM, CS, 16, 6, 1>(a, ngroups, st);
            case 7: return launch_team<BITS, SYM, CS, 16, 7, 1>(a, ngroups, st);
            default: return launch_team<BITS, SYM, CS, 16, 8, 1>(a, ngroups, st);
        }
    } else if (CS && a.group == a.k && a.k <= kBigLoads * 256 * 8) {
        if (a.k >= 6144)
            hipLaunchKernelGGL((quant_rows_cs_kernel<BITS, SYM, 2>), dim3((uint32_t)((a.n + 1) / 2)), dim3(256), 0, st,
                               a.w, a.n, a.k, a.col_scale, a.codes, a.scales, a.zeros);
        else
            hipLaunchKernelGGL((quant_rows_cs_kernel<BITS, SYM, 1>), dim3((uint32_t)a.n), dim3(256), 0, st, a.w, a.n,
                               a.k, a.col_scale, a.codes, a.scales, a.zeros);
    } else if (a.group <= kBigLoads * 256 * 8) {
        hipLaunchKernelGGL((quant_big_kernel<BITS, SYM, CS, true, 256>), dim3((uint32_t)ngroups), dim3(256), 0, st,
                           a.w, a.group, a.k, a.col_scale, a.codes, a.scales, a.zeros);
    } else if (a.group <= kBigLoads * 1024 * 8) {
        hipLaunchKernelGGL((quant_big_kernel<BITS, SYM, CS, true, 1024>), dim3((uint32_t)ngroups), dim3(1024), 0,
                           st, a.w, a.group, a.k, a.col_scale, a.codes, a.scales, a.zeros);
    } else {
        hipLaunchKernelGGL((quant_big_kernel<BITS, SYM, CS, false, 1024>), dim3((uint32_t)ngroups), dim3(1024), 0,
                           st, a.w, a.group, a.k, a.col_scale, a.codes, a.scales, a.zeros);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st) {
    const bool cs = a.col_scale != nullptr;
#define LQ_Q(B, S)                                                              \
    if (a.bits == B && (a.symmetric != 0) == S)                                 \
        return cs ? launch_quant_t<B, S, true>(a, st) : launch_quant_t<B, S, false>(a, st);
    LQ_Q(4, true) LQ_Q(4, false) LQ_Q(8, true) LQ_Q(8, false)
#undef LQ_Q
    return hipErrorInvalidValue;
}

template <int BITS, bool SYM>
static hipError_t launch_dequant_t(const DequantArgs &a, hipStream_t st) {
    const int64_t total = a.n * a.k;
    const int64_t blocks = (total + 2047) / 2048;
    hipLaunchKernelGGL((dequant_kernel<BITS, SYM>), dim3((uint32_t)blocks), dim3(256), 0, st,
                       a.codes, a.scales, a.zeros, total, a.group, a.out);
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t st) {
    if (a.bits == 4) return a.symmetric ? launch_dequant_t<4, true>(a, st) : launch_dequant_t<4, false>(a, st);
    return a.symmetric ? launch_dequant_t<8, true>(a, st) : launch_dequant_t<8, false>(a, st);
}

}  // namespace lq
