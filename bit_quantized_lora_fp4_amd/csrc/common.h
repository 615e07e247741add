// Device helpers shared by the gfx950 kernels: vector types, MXFP4 scale rule,
// hardware E2M1 conversion, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef uint16_t bf16_t;  // raw bf16 bits in memory

// ---------------------------------------------------------------- MXFP4 block scale
// Shared exponent of a 32x32 block (FourTune §2.3 names MXFP4; the MX rule is
// E = floor(log2 amax) - 2 for E2M1, clamped to [-127, 127], stored biased by 127).
// `amax_bits` is the fp32 bit pattern of max|x| over the block (sign bit clear).
// For a normal amax, floor(log2 amax) = biased exponent - 127, so the stored byte is
// biased_exp - 2; subnormal or zero amax, and biased_exp <= 2, clamp to byte 0. An
// exponent field of 255 means the block held a NaN or infinity: byte 0xFF.
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  uint32_t e = amax_bits >> 23;
  if (e == 255u) return 0xFFu;
  return e > 2u ? e - 2u : 0u;
}

// fp32 whose exponent field is the E8M0 byte: the form the hardware conversions take
// as their scale (the byte's value is 2^(byte-127); byte 0 maps to bits 0).
__device__ __forceinline__ float e8m0_to_f32_scale(uint32_t byte) {
  return __builtin_bit_cast(float, byte << 23);
}

// ---------------------------------------------------------------- E2M1 conversion
// v_cvt_scalef32_pk_fp4_{bf16,f32}: two values divided by the scale and rounded to
// nearest E2M1 (ties to even code, saturating at +-6, sign of zero kept), packed into
// byte `sel` of the result. Verified against the quantizer's definition on every bf16
// pattern under every scale byte.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// 8 bf16 values (4 words, even element in the low half) -> 8 codes in one word.
__device__ __forceinline__ uint32_t cvt8_bf16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                              float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w3), scale, 3);
  return r;
}

// 8 fp32 values -> 8 codes in one word.
__device__ __forceinline__ uint32_t cvt8_f32(const float* v, float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], scale, 3);
  return r;
}

// ---------------------------------------------------------------- bf16 helpers
// fp32 -> bf16 round-to-nearest-even on the bit pattern (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// max of the two 15-bit magnitudes held in a bf16 pair word, as fp32 bits
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
  return (a > b ? a : b) << 16;
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int MASK>
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v) {
  return (uint32_t)__shfl_xor((int)v, MASK, 64);
}

}  // namespace ft
