// Matrix-core operand helpers for gfx950 shared by the decode and prefill attention kernels:
// v_mfma_f32_16x16x32_f16 with exact code operands (packed cache codes turned into fp16 bit
// patterns without a conversion), fp16 hi / lo operand pairs, and reductions over a DPP row.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {
namespace mops {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// An operand x goes in as fp16 hi = fp16(x) plus lo = fp16((x - hi) * 2^11): the scaled low part
// stays a normal fp16 number whenever hi is, so the pair keeps about 22 significant bits; the
// products of the lo parts are scaled back by 2^-11.
constexpr float kLoScale = 2048.0f, kLoInv = 1.0f / 2048.0f;

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8 as_h8(u4 v) { return __builtin_bit_cast(h8, v); }
__device__ __forceinline__ float c0f() { return __uint_as_float(0x3DB504F3u); }
__device__ __forceinline__ float lo_h(uint32_t w) { return (float)__builtin_bit_cast(h2v, w)[0]; }
__device__ __forceinline__ float hi_h(uint32_t w) { return (float)__builtin_bit_cast(h2v, w)[1]; }

// (x & m) | c as one v_and_or_b32.  Written plainly, the compiler emits an AND and an OR, each
// with its own literal (a three-operand instruction takes no literal on this architecture), so
// the operand builders below that mask code bits and set an fp16 exponent cost two instructions
// per word instead of one.  m is a wave-uniform constant (scalar register), c a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
}

// 4-bit word (channel/token i at bit 16*(i%2) + 4*(i/2)) -> 8 fp16 subnormal operands in
// natural order, slots 2,3,6,7 carry an extra factor 16.
__device__ __forceinline__ u4 unpack4(uint32_t x) {
    u4 r;
    r.x = x & 0x000F000Fu;
    r.y = x & 0x00F000F0u;
    const uint32_t y = x >> 8;
    r.z = y & 0x000F000Fu;
    r.w = y & 0x00F000F0u;
    return r;
}

// 8 bytes (value i at byte i) -> 8 zero-extended 16-bit operands in natural order.
__device__ __forceinline__ u4 unpack8(uint32_t x0, uint32_t x1) {
    u4 r;
    r.x = __builtin_amdgcn_perm(0u, x0, 0x0c010c00u);
    r.y = __builtin_amdgcn_perm(0u, x0, 0x0c030c02u);
    r.z = __builtin_amdgcn_perm(0u, x1, 0x0c010c00u);
    r.w = __builtin_amdgcn_perm(0u, x1, 0x0c030c02u);
    return r;
}

// V operands are centred so that no large one-signed sum has to cancel against the zero-point
// term: a code c enters as the exact fp16 integer c - 8 (4-bit) or c - 128 (8-bit), made by
// placing c in the mantissa of 1024 (bit pattern 0x6400 | c) and subtracting 1024 + 8 (or the
// x16 slots' 1024 + 128, or 1024 + 128 for 8-bit codes) with one packed fp16 add.
__device__ __forceinline__ uint32_t h2sub(uint32_t x, _Float16 c) {
    const h2v r = __builtin_bit_cast(h2v, x) - h2v{c, c};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ u4 centred4(uint32_t x) {
    u4 r;
    r.x = h2sub(and_or(x, 0x000F000Fu, 0x64006400u), (_Float16)1032.0f);
    r.y = h2sub(and_or(x, 0x00F000F0u, 0x64006400u), (_Float16)1152.0f);
    const uint32_t y = x >> 8;
    r.z = h2sub(and_or(y, 0x000F000Fu, 0x64006400u), (_Float16)1032.0f);
    r.w = h2sub(and_or(y, 0x00F000F0u, 0x64006400u), (_Float16)1152.0f);
    return r;
}
__device__ __forceinline__ u4 centred8(uint32_t x0, uint32_t x1) {
    const u4 b = unpack8(x0, x1);
    u4 r;
    r.x = h2sub(b.x | 0x64006400u, (_Float16)1152.0f);
    r.y = h2sub(b.y | 0x64006400u, (_Float16)1152.0f);
    r.z = h2sub(b.z | 0x64006400u, (_Float16)1152.0f);
    r.w = h2sub(b.w | 0x64006400u, (_Float16)1152.0f);
    return r;
}
// Reductions across the 16 lanes of a DPP row (lanes 16r .. 16r+15): swap within pairs, within
// quads, mirror within half-rows, mirror within the row; every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v)); // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v)); // row_mirror
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}


} // namespace mops
} // namespace kvq
