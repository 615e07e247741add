// Device helpers shared by the gfx950 kernels: vector types, MXFP4 scale rule,
// hardware E2M1 conversion, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
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
// fp32 -> bf16, round to nearest even (NaN kept quiet): the gfx950 conversion
// v_cvt_pk_bf16_f32, which the compiler emits for a float2 -> bf16x2 vector conversion.
// Checked bit for bit against the integer formulation (bias 0x7FFF plus the kept bit's
// parity, then truncation) on 16.7M patterns including ties, denormals and NaNs.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// max of the two 15-bit magnitudes held in a bf16 pair word, as fp32 bits
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
  return (a > b ? a : b) << 16;
}

// ---------------------------------------------------------------- GELU (tanh form)
// GELU(p) = p/2 (1 + tanh(u)), u = sqrt(2/pi) (p + 0.044715 p^3) (FourTune §3.3 "MLP
// Fusion" applies GELU between the two linears of an MLP), evaluated without
// cancellation as p * s with s = (1 + tanh(u))/2 = 1 / (1 + e^(-2u)); e^(-2u) comes from
// the hardware base-2 exponential and s from the hardware reciprocal, so the relative
// error stays within a few fp32 ulps also where GELU is tiny (large negative p).
// Derivative: s + p (1 - tanh^2(u))/2 du/dp = s (1 + 2 p (1 - s) du/dp).
// Large |u| saturates correctly (e -> 0 or inf); NaN propagates.
constexpr double GELU_K0 = 0.7978845608028654;  // sqrt(2/pi)
constexpr double GELU_K1 = 0.044715;
constexpr double LN_2 = 0.6931471805599453;
// -2u / ln 2 = p (A0 + A1 p^2): the exponent of e^(-2u) in base 2
constexpr float GELU_A0 = (float)(-2.0 * GELU_K0 / LN_2);
constexpr float GELU_A1 = (float)(-2.0 * GELU_K0 * GELU_K1 / LN_2);
// 2 du/dp = B0 + B1 p^2
constexpr float GELU_B0 = (float)(2.0 * GELU_K0);
constexpr float GELU_B1 = (float)(6.0 * GELU_K0 * GELU_K1);
__device__ __forceinline__ float gelu_f(float p) {
  const float e = __builtin_amdgcn_exp2f(p * __builtin_fmaf(GELU_A1, p * p, GELU_A0));
  return p * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_grad_f(float p) {
  const float p2 = p * p;
  const float e = __builtin_amdgcn_exp2f(p * __builtin_fmaf(GELU_A1, p2, GELU_A0));
  const float sg = __builtin_amdgcn_rcpf(1.0f + e);
  // 1 - s, formed without overflow (e may be huge or infinite) or cancellation
  const float es = e > 1.0f ? 1.0f - sg : e * sg;
  float g = sg * __builtin_fmaf(p * es, __builtin_fmaf(GELU_B1, p2, GELU_B0), 1.0f);
  // |p| > 16: the derivative is 1 (or 0) to fp32 precision; p^3 may overflow there.
  // g is pinned as computed, so the choice stays a select rather than a branch around
  // the arithmetic (a branch per element costs more than the arithmetic it skips).
  asm volatile("" : "+v"(g));
  return fabsf(p) > 16.0f ? (p > 0.0f ? 1.0f : 0.0f) : g;
}
// 8 bf16 (4 words) -> bf16(GELU(x)) for each, rounded to nearest even
__device__ __forceinline__ uint32_t gelu_bf16x2(uint32_t w) {
  return pack_bf16x2(gelu_f(bf16_lo(w)), gelu_f(bf16_hi(w)));
}

// ---------------------------------------------------------------- LDS transposed reads
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4s __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, source lane s supplies the address of
// 4 consecutive 16-bit elements; viewing the group's 64 elements as 4 rows of 16 (row q
// = source lanes 4q..4q+3), output lane i receives column i of those 4 rows.
// lds_tr16_pair reads, from a row-major bf16 tile (row pitch `pitch` bytes), the bf16
// MFMA operand "8 consecutive rows m0 + 8*(l/32) .. +8 of column c0 + l%32" for every
// lane l, as two such reads.
__device__ __forceinline__ v4i lds_tr16_pair(const lds_char* base, int pitch, int m0, int c0, int lane) {
  // 8 consecutive m (m0 + 8*(l>>5) .. +8) of column c0 + (l & 31), via two tr_b16 reads
  const int g = lane >> 4, s = lane & 15;
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int m = m0 + 8 * (g >> 1) + (s >> 2);
  const lds_char* p0 = base + m * pitch + col * 2;
  v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
  v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0 + 4 * pitch));
  v4i r;
  r.x = (int)(((uint32_t)(uint16_t)lo.x) | ((uint32_t)(uint16_t)lo.y << 16));
  r.y = (int)(((uint32_t)(uint16_t)lo.z) | ((uint32_t)(uint16_t)lo.w << 16));
  r.z = (int)(((uint32_t)(uint16_t)hi.x) | ((uint32_t)(uint16_t)hi.y << 16));
  r.w = (int)(((uint32_t)(uint16_t)hi.z) | ((uint32_t)(uint16_t)hi.w << 16));
  return r;
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources: loads beyond num_records bytes return zero with no branch, so
// ragged tiles need no predicated code. An offset of BUF_OOB is always out of range.
typedef __amdgpu_buffer_rsrc_t bufres;
constexpr uint32_t BUF_OOB = 0xFFFFFF00u;
constexpr int BUF_FLAGS = 0x00020000;  // raw, untyped 32-bit data (gfx9 dword3)

__device__ __forceinline__ bufres make_buf(const void* base, uint64_t bytes) {
  const uint32_t n = bytes >= 0xFFFFFF00ull ? 0xFFFFFF00u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, BUF_FLAGS);
}
__device__ __forceinline__ v4i buf_load16(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
__device__ __forceinline__ v2i buf_load8(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(bufres r, uint32_t off, v2i v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(bufres r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(bufres r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store1(bufres r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, (int)off, 0, 0);
}
// `ok ? off : BUF_OOB`, kept opaque so that the optimizer does not turn the select
// into control flow around the load that consumes it.
__device__ __forceinline__ uint32_t sel_off(bool ok, uint32_t off) {
  uint32_t v = ok ? off : BUF_OOB;
  asm("" : "+v"(v));
  return v;
}
// 16 bytes per lane straight into LDS: lane l's data lands at lds + 16*l.
__device__ __forceinline__ void buf_load16_lds(bufres r, lds_char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)off, 0, 0, 0);
}
// Nontemporal forms (cache-policy operand NT = 2): for data read or written once, so
// it streams past the caches instead of displacing what is reused.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ void buf_load16_lds_nt(bufres r, lds_char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)off, 0, 0, CPOL_NT);
}
__device__ __forceinline__ v4i buf_load16_nt(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL_NT);
}
__device__ __forceinline__ void buf_store16_nt(bufres r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, CPOL_NT);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int MASK>
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v) {
  return (uint32_t)__shfl_xor((int)v, MASK, 64);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the 64 lanes, all in VALU: DPP butterflies inside each 16-lane row,
// then v_permlane16_swap / v_permlane32_swap, each of which leaves a lane holding its
// own value and that of lane ^16 (^32) in its two results.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = umax(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = umax(v, dpp<0x141>(v));  // row_half_mirror: the other quad of the 8
  v = umax(v, dpp<0x140>(v));  // row_mirror: the other half of the row
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax(p[0], p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(q[0], q[1]);
}

// p[0] + p[stride] + ... + p[(S-1) stride] (S >= 1), added in range order. The loads
// go out in batches of four before any add waits, so the ranges cost one memory round
// trip per batch instead of one per range: a batch's loads past the last range repeat
// the last range's address (no branches, which would make the compiler wait at each
// one), and the adds of those are selected away.
__device__ __forceinline__ v4f sum_ranges(const v4f* __restrict__ p, int S, int64_t stride) {
  v4f s = p[0];
  for (int b = 1; b < S; b += 4) {
    v4f t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = p[(int64_t)min(b + u, S - 1) * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const v4f n = s + t[u];
      s = b + u < S ? n : s;
    }
  }
  return s;
}

}  // namespace ft
