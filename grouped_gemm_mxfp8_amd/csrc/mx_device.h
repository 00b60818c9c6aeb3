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

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950 converts two
// values in one v_cvt_pk_bf16_f32 (equal, for every non-NaN fp32 pattern, to
// the integer rounding u + 0x7fff + ((u >> 16) & 1), checked exhaustively on
// the device).  bf16x2 packs a in the low and b in the high half.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return bf16x2(f, 0.0f) & 0xffffu;
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

// E4M3 codes of four values, each multiplied by its block's 2^-X first (an
// exact power-of-two scaling), packed into one dword (byte k = value k).
// The hardware conversion v_cvt_pk_fp8_f32 rounds to nearest even and keeps
// the sign of values that round to zero; the med3 clamp to +-448 beforehand
// makes out-of-range values saturate instead of becoming NaN.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float ia,
                                           float ib, float ic, float id) {
    a = __builtin_amdgcn_fmed3f(a * ia, 448.0f, -448.0f);
    b = __builtin_amdgcn_fmed3f(b * ib, 448.0f, -448.0f);
    c = __builtin_amdgcn_fmed3f(c * ic, 448.0f, -448.0f);
    d = __builtin_amdgcn_fmed3f(d * id, 448.0f, -448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
    return e4m3x4(a, b, c, d, inv, inv, inv, inv);
}

// The block scale 2^X = 2^(c - 127) of E8M0 code c (c = 0 gives the fp32
// subnormal 2^-127; these kernels keep fp32 denormals).
__device__ __forceinline__ float scale_from_code(uint32_t c) {
    return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)c);
}
// 448 * 2^X for code c: 1.75 * 2^(c - 119), a normal number for every c.
__device__ __forceinline__ float e4m3_limit_from_code(uint32_t c) {
    return __uint_as_float(((c + 8u) << 23) | 0x600000u);
}

typedef short v2s16 __attribute__((ext_vector_type(2)));
// E4M3 codes of a and b divided by a block scale, in the low (hi = false) or
// high half of old: v_cvt_scalef32_pk_fp8_f32 divides by the scale (exact, a
// power of two) and rounds to nearest even but does not saturate, so the
// values are clamped to +-lim = +-448 * scale first.  Equal, code for code, to
// clamping x * 2^-X to +-448 and converting (checked on the device over every
// finite bf16 pattern and random fp32 values at scale exponents from -127 to
// 30).
__device__ __forceinline__ uint32_t e4m3x2_scaled(uint32_t old, float a, float b, float lim,
                                                  float scale, bool hi) {
    a = __builtin_amdgcn_fmed3f(a, lim, -lim);
    b = __builtin_amdgcn_fmed3f(b, lim, -lim);
    const v2s16 o = __builtin_bit_cast(v2s16, old);
    const v2s16 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, false);
    return __builtin_bit_cast(uint32_t, r);
}
// Four values of one block: bytes a, b, c, d.  The first conversion writes
// the low half and the second the high half, so the first one's other half
// may be anything: a's own bits, whose register the conversion can then
// write in place (a zero there would cost a register copy per dword).
__device__ __forceinline__ uint32_t e4m3x4_scaled(float a, float b, float c, float d, float lim,
                                                  float scale) {
    return e4m3x2_scaled(e4m3x2_scaled(__float_as_uint(a), a, b, lim, scale, false), c, d, lim,
                         scale, true);
}

// Streaming stores: the output is read by a later kernel, never again by
// this one, so the nontemporal hint keeps it from displacing lines that the
// running kernels re-read from the caches.
__device__ __forceinline__ void store_nt(void* p, uint4 v) {
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((u32x4_nt){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_nt*>(p));
}
__device__ __forceinline__ void store_nt(void* p, uint2 v) {
    typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store((u32x2_nt){v.x, v.y}, reinterpret_cast<u32x2_nt*>(p));
}

// Max of |v| as fp32 bit pattern (non-negative floats order like integers).
__device__ __forceinline__ uint32_t abs_bits(float v) {
    return __float_as_uint(v) & 0x7fffffffu;
}

}  // namespace mx
