// Device helpers of the MXFP8 MoE expert path (gfx950 only).
//
// Encoding (the MXFP8 paragraphs of the three pages: 8-bit values with one
// scale per block of 32): elements are OCP E4M3 (bias 7, no infinities,
// S.1111.111 is NaN, largest finite 448 = 0x7E); scales are E8M0 (code c is
// 2^(c-127)).  The scale exponent of a block is X = floor(log2(amax)) - 8
// clamped to [-127, 127] (X = -127 for an all-zero block); elements are
// v * 2^-X rounded to nearest even and saturated at +-448, the sign kept for
// values that round to zero.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// E8M0 scale code of a block from the bit pattern of its (non-negative,
// finite) amax as fp32: X + 127 = biased exponent - 8, floored at 0.  A zero
// or subnormal amax has biased exponent 0 and gives code 0 (X = -127).
__device__ __forceinline__ uint32_t scale_code_from_amax_bits(uint32_t amax_bits) {
    int e = (int)(amax_bits >> 23) - 8;
    return e < 0 ? 0u : (uint32_t)e;
}

// 2^-X as fp32 for scale code c = X + 127 (always a normal number: c <= 246
// for finite inputs, so 254 - c >= 8).
__device__ __forceinline__ float inv_scale_from_code(uint32_t c) {
    return __uint_as_float((254u - c) << 23);
}

// E4M3 code of a non-negative finite magnitude a (already divided by the
// block scale), RNE, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_from_mag(float a) {
    if (a >= 448.0f) return 0x7eu;
    if (a < 0.015625f)                        // below 2^-6: subnormal grid 2^-9
        return (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8 (8 -> 0x08)
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);         // RNE to 3 mantissa bits
    uint32_t c = (u >> 20) - (120u << 3);     // rebias exponent 127 -> 7
    return c > 0x7eu ? 0x7eu : c;             // a < 448 never exceeds 0x7E
}

// E4M3 code of v * inv_scale with v's sign kept.
__device__ __forceinline__ uint32_t e4m3_encode(float v, float inv_scale) {
    uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
    return s | e4m3_from_mag(__builtin_fabsf(v) * inv_scale);
}

// Max of |v| as fp32 bit pattern (non-negative floats order like integers).
__device__ __forceinline__ uint32_t abs_bits(float v) {
    return __float_as_uint(v) & 0x7fffffffu;
}

}  // namespace mx
