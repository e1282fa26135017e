// Weight-code decoding and MFMA helpers shared by the projection kernels
// (verify and prefill): every quantised code becomes an exact bf16 value, so
// the matrix cores contract codes and bf16 activations without rounding.
#pragma once

#include "dspk_internal.h"

namespace dspk {
namespace dec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// high halves of two floats holding small integers -> one dword of two bf16 (exact)
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// eight 8-bit codes (two dwords, LSB first) -> eight exact bf16 values, same order
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r[0] = pack_hi16((float)(w0 & 0xffu), (float)((w0 >> 8) & 0xffu));
    r[1] = pack_hi16((float)((w0 >> 16) & 0xffu), (float)(w0 >> 24));
    r[2] = pack_hi16((float)(w1 & 0xffu), (float)((w1 >> 8) & 0xffu));
    r[3] = pack_hi16((float)((w1 >> 16) & 0xffu), (float)(w1 >> 24));
    return as_bf16x8(r);
}

// The constant 0x43004300 (two bf16 128.0) in a vector register, opaque to
// the compiler.  A gfx9 VOP3 instruction reads at most one scalar or literal
// operand, so with the mask and this constant both literal the compiler
// splits (x & mask) | c into an and and an or; with c in a vector register
// it forms one v_and_or_b32.  Only ordinary VALU instructions read the
// result.
__device__ __forceinline__ uint32_t bf16_128_pair() {
    uint32_t r;
    asm("v_mov_b32 %0, 0x43004300" : "=v"(r));
    return r;
}
// eight 4-bit codes (one dword) -> bf16 values 128 + q in the order
// q0,q4,q1,q5,q2,q6,q3,q7 (0x4300 is bf16 128.0; q fills the low mantissa bits)
__device__ __forceinline__ bf16x8 codes4_to_bf16(uint32_t w) {
    const uint32_t c = bf16_128_pair();
    u32x4 r;
    r[0] = (w & 0x000F000Fu) | c;
    r[1] = ((w >> 4) & 0x000F000Fu) | c;
    r[2] = ((w >> 8) & 0x000F000Fu) | c;
    r[3] = ((w >> 12) & 0x000F000Fu) | c;
    return as_bf16x8(r);
}

// sixteen 2-bit codes (one dword, code e in bits 2e..2e+1) -> two bf16x8 of
// 128 + q in the order q0,q8,q1,q9,q2,q10,q3,q11 | q4,q12,...,q7,q15
__device__ __forceinline__ void codes2_to_bf16(uint32_t w, bf16x8 &b0, bf16x8 &b1) {
    u32x4 r0, r1;
    const uint32_t c = bf16_128_pair();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r0[i] = ((w >> (2 * i)) & 0x00030003u) | c;
        r1[i] = ((w >> (2 * i + 8)) & 0x00030003u) | c;
    }
    b0 = as_bf16x8(r0);
    b1 = as_bf16x8(r1);
}

// sixteen 3-bit codes: low planes as for 2-bit (lo) and the high bits h with
// code e's at bit e (e < 8) and at bit 16 + e - 8 (e >= 8), so that the bit of
// code i lands at bit 2 of a half and that of code i + 8 at bit 18
__device__ __forceinline__ void codes3_to_bf16(uint32_t lo, uint32_t h, bf16x8 &b0, bf16x8 &b1) {
    u32x4 r0, r1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r0[i] = ((lo >> (2 * i)) & 0x00030003u) | ((((h >> i) << 2) & 0x00040004u) | 0x43004300u);
        r1[i] = ((lo >> (2 * i + 8)) & 0x00030003u) | ((((h >> (i + 4)) << 2) & 0x00040004u) | 0x43004300u);
    }
    b0 = as_bf16x8(r0);
    b1 = as_bf16x8(r1);
}

// activations x0..x7 (p0) and x8..x15 (p1) reordered to match codes2_to_bf16
__device__ __forceinline__ void perm_x_for2(u32x4 p0, u32x4 p1, u32x4 &a0, u32x4 &a1) {
    a0[0] = __builtin_amdgcn_perm(p1[0], p0[0], 0x05040100u);
    a0[1] = __builtin_amdgcn_perm(p1[0], p0[0], 0x07060302u);
    a0[2] = __builtin_amdgcn_perm(p1[1], p0[1], 0x05040100u);
    a0[3] = __builtin_amdgcn_perm(p1[1], p0[1], 0x07060302u);
    a1[0] = __builtin_amdgcn_perm(p1[2], p0[2], 0x05040100u);
    a1[1] = __builtin_amdgcn_perm(p1[2], p0[2], 0x07060302u);
    a1[2] = __builtin_amdgcn_perm(p1[3], p0[3], 0x05040100u);
    a1[3] = __builtin_amdgcn_perm(p1[3], p0[3], 0x07060302u);
}

// eight bf16 activations reordered to match codes4_to_bf16
__device__ __forceinline__ u32x4 perm_x_for4(u32x4 x) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);
    return r;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f2bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Unit geometry of a weight format: KU K elements per unit, GS = KU / 64
// groups, SBQ 16-byte scale/bias loads per lane (one per group: the dwords of
// the lane's four column tiles), UNIT bytes per unit.
template <int BITS>
struct Cfg {
    static constexpr int KU = tile_k(BITS);
    static constexpr int GS = tile_groups(BITS);
    static constexpr int SBQ = BITS == 16 ? 0 : GS;
    static constexpr int UNIT = tile_unit_bytes(BITS);
    static constexpr int NS = tile_code_slots(BITS);     // 1 KiB code slots per unit
    static constexpr int SBOFF = 1024 * NS;              // scale/bias dwords within a unit
};

}  // namespace dec
}  // namespace dspk
