// common.hpp -- small device helpers shared by the gfx950 kernels of libquant.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LQ_DEVICE __device__ __forceinline__

namespace lq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact: bf16 is the upper half of an fp32).
LQ_DEVICE float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
LQ_DEVICE float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The pages' clamp(min = 1e-8) floor on a range or absmax before the division.
constexpr float kFloor = 1e-8f;

// Same comparison order as the definition: below lo -> lo, above hi -> hi.
LQ_DEVICE float clamp_code(float v, float lo, float hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Butterfly sum / max over `width` lanes (width a power of two, <= 64).
template <int WIDTH>
LQ_DEVICE float team_sum(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WIDTH);
    return v;
}
template <int WIDTH>
LQ_DEVICE float team_max(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WIDTH));
    return v;
}
template <int WIDTH>
LQ_DEVICE float team_min(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, WIDTH));
    return v;
}

// DPP lane moves inside rows of 16 lanes (gfx9 DPP control codes)
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16 lanes

template <int CTRL>
LQ_DEVICE float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}


// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3).
// Loads whose offset falls outside return zeros instead of faulting.
LQ_DEVICE __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past any resource used here
constexpr int kNonTemporal = 2;                // buffer-load cache policy: streaming

// INT4 code word (element i at bits 4i..4i+3) -> 4 packed bf16 pairs
// (128 + c_2i, 128 + c_2i+1), natural k order: byte i of the word gives the
// low half, byte i of the word shifted right by 4 the high half. A nibble
// ORed into the mantissa of bf16 128 is exactly 128 + c. `magic` holds the
// bf16 pair (128, 128) = 0x43004300 (passed in a VGPR so the masking selects
// v_and_or_b32).
LQ_DEVICE u32x4 unpack_natural(uint32_t w, uint32_t magic) {
    const uint32_t w4 = w >> 4;
    u32x4 p;
    p.x = (__builtin_amdgcn_perm(w4, w, 0x0C040C00u) & 0x000F000Fu) | magic;
    p.y = (__builtin_amdgcn_perm(w4, w, 0x0C050C01u) & 0x000F000Fu) | magic;
    p.z = (__builtin_amdgcn_perm(w4, w, 0x0C060C02u) & 0x000F000Fu) | magic;
    p.w = (__builtin_amdgcn_perm(w4, w, 0x0C070C03u) & 0x000F000Fu) | magic;
    return p;
}

// fp32 quotient a / b from y = RN(1 / b) and FMA corrections (Markstein's
// division; Muller et al., Handbook of Floating-Point Arithmetic, division
// with a fused multiply-add): the first correction leaves q1 within one ulp
// of a / b, and for such a q1 the step RN(q1 + (a - b q1) y), with the
// residual exact, is RN(a / b), the IEEE quotient. That holds while every
// intermediate is normal and finite; each caller states why its operands
// qualify.
LQ_DEVICE float div_rn(float a, float b, float y) {
    const float q0 = a * y;
    const float r0 = __builtin_fmaf(-q0, b, a);
    const float q1 = __builtin_fmaf(r0, y, q0);
    const float r1 = __builtin_fmaf(-q1, b, a);
    return __builtin_fmaf(r1, y, q1);
}

// Workgroup barrier ordering LDS accesses only. __syncthreads() also
// releases global memory, which makes each wave wait for all of its
// outstanding global loads; this one leaves prefetches in flight.
LQ_DEVICE void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// v_dot2_f32_bf16: acc + a.lo * b.lo + a.hi * b.hi, with both pairs passed
// as packed 32-bit words.
LQ_DEVICE float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Transposed exchange across lane halves of width 32 (or 16): afterwards the
// lanes of the lower half hold a + (partner's a), those of the upper half
// b + (partner's b). v_permlane{32,16}_swap trades the upper half of its
// first operand for the lower half of its second.
LQ_DEVICE float swap_add32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
LQ_DEVICE float swap_add16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum RW (4 or 8) values per lane over the 64 lanes of a wave. Each halving
// step sends half of the remaining values to the partner lane (lane bits 5,
// 4, then 3), plain butterflies finish the rest. Afterwards every lane l
// holds the total of row l >> (6 - log2 RW).
template <int RW>
LQ_DEVICE float reduce_rows(float *v, int lane) {
    static_assert(RW == 4 || RW == 8, "RW must be 4 or 8");
#pragma unroll
    for (int i = 0; i < RW / 2; ++i) v[i] = swap_add32(v[i], v[i + RW / 2]);
#pragma unroll
    for (int i = 0; i < RW / 4; ++i) v[i] = swap_add16(v[i], v[i + RW / 4]);
    float t = v[0];
    if (RW == 8) {
        // partner lane l ^ 15 sits across bit 3: lanes with bit 3 clear keep row 0 of the pair
        const bool upper = (lane & 8) != 0;
        const float keep = upper ? v[1] : v[0];
        const float send = upper ? v[0] : v[1];
        t = keep + dpp_move<kDppMirror>(send);
    } else {
        t += dpp_move<kDppMirror>(t);
    }
    t += dpp_move<kDppHalfMirror>(t);
    t += dpp_move<kDppXor2>(t);
    t += dpp_move<kDppXor1>(t);
    return t;
}

}  // namespace lq
