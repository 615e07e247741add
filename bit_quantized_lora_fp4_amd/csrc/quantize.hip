// Standalone 32x32-block MXFP4 quantizer (FourTune §2.3 quantizer form with group
// scales; §3.2 block-wise quantization with block-local scales).
//
// HBM-bound: per element it reads 2 bytes (bf16) or 4 (fp32) and writes half a byte
// of code, plus one scale byte per 1024 elements.
//
// Mapping. A wave owns a 32-row x 128-column tile (four 32x32 blocks). Lane l covers
// columns 8*(l%16) .. +8 of the tile and rows 4*i + l/16 (i = 0..7), so each load
// instruction reads 4 rows x 256 contiguous bytes (bf16) and every lane keeps all of
// its 8 loads in flight before any arithmetic. The 16 lanes sharing a block (same
// (l%16)/4) combine their maxima with four butterfly steps (lane masks 1, 2, 16, 32).
// Each lane then converts its 64 values with the hardware E2M1 conversion and writes
// one 32-bit word (8 codes) per row: 16 lanes write 64 contiguous bytes of a row.
//
// GROUPS = true is the 1x32 form (one scale per row and 32 columns, the granularity
// FourTune §4 "Impact of Quantization Granularity" compares the blocks against): the
// same mapping, the maximum taken per row over the 4 lanes of a group (masks 1, 2),
// scales stored [rows x cols/32].
#include "common.h"

namespace ft {

template <typename T>
struct QuantIO;

// 16 bytes; NT: nontemporal (streamed past the caches)
template <bool NT>
__device__ __forceinline__ v4i load16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  else return *reinterpret_cast<const v4i*>(p);
}

template <>
struct QuantIO<bf16_t> {
  static constexpr int WORDS = 4;  // 8 bf16 per lane-row = 16 bytes
  template <bool NT>
  __device__ static void load(const bf16_t* p, bool ok, uint32_t* w) {
    const v4i v = ok ? load16<NT>(p) : v4i{0, 0, 0, 0};
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ static uint32_t absmax(const uint32_t* w) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = umax(m, bf16x2_absmax_bits(w[j]));
    return m;
  }
  __device__ static uint32_t codes(const uint32_t* w, float scale) {
    return cvt8_bf16(w[0], w[1], w[2], w[3], scale);
  }
};

template <>
struct QuantIO<float> {
  static constexpr int WORDS = 8;  // 8 fp32 per lane-row = 32 bytes
  template <bool NT>
  __device__ static void load(const float* p, bool ok, uint32_t* w) {
    const v4i a = ok ? load16<NT>(p) : v4i{0, 0, 0, 0};
    const v4i b = ok ? load16<NT>(p + 4) : v4i{0, 0, 0, 0};
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ static uint32_t absmax(const uint32_t* w) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, w[j] & 0x7FFFFFFFu);
    return m;
  }
  __device__ static uint32_t codes(const uint32_t* w, float scale) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = __builtin_bit_cast(float, w[j]);
    return cvt8_f32(f, scale);
  }
};

template <typename T, bool GROUPS, bool NT>
__global__ __launch_bounds__(256) void k_quantize(const T* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t ld,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  using IO = QuantIO<T>;
  const int lane = threadIdx.x & 63;
  const int64_t c0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 128;
  if (c0 >= cols) return;  // wave-uniform
  const int64_t r0 = (int64_t)blockIdx.y * 32;
  const int sub = lane & 15, rq = lane >> 4;
  const int64_t col = c0 + sub * 8;
  const bool col_ok = col < cols;  // cols % 32 == 0: an 8-column group is all in or out

  uint32_t w[8][IO::WORDS];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = r0 + 4 * i + rq;
    IO::template load<NT>(x + row * ld + col, col_ok && row < rows, w[i]);
  }
  if constexpr (GROUPS) {
    const int64_t cpitch = cols >> 1, spitch = cols >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = r0 + 4 * i + rq;
      uint32_t m = IO::absmax(w[i]);
      m = umax(m, shfl_xor_u32<1>(m));
      m = umax(m, shfl_xor_u32<2>(m));
      const uint32_t sb = scale_byte_from_amax(m);
      uint32_t c = IO::codes(w[i], e8m0_to_f32_scale(sb));
      if (sb == 0xFFu) c = 0;  // non-finite group: zero codes
      if (col_ok && row < rows) {
        *reinterpret_cast<uint32_t*>(codes + row * cpitch + (col >> 1)) = c;
        if ((sub & 3) == 0) scales[row * spitch + (col >> 5)] = (uint8_t)sb;
      }
    }
    return;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = umax(amax, IO::absmax(w[i]));
  amax = umax(amax, shfl_xor_u32<1>(amax));
  amax = umax(amax, shfl_xor_u32<2>(amax));
  amax = umax(amax, shfl_xor_u32<16>(amax));
  amax = umax(amax, shfl_xor_u32<32>(amax));
  const uint32_t sb = scale_byte_from_amax(amax);
  const float scale = e8m0_to_f32_scale(sb);
  if (!col_ok) return;

  const int64_t cpitch = cols >> 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = r0 + 4 * i + rq;
    uint32_t c = IO::codes(w[i], scale);
    if (sb == 0xFFu) c = 0;  // non-finite block: zero codes
    if (row < rows) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * cpitch + (col >> 1));
      if constexpr (NT) __builtin_nontemporal_store(c, dst);
      else *dst = c;
    }
  }
  if (rq == 0 && (sub & 3) == 0) scales[(int64_t)blockIdx.y * (cols >> 5) + (col >> 5)] = (uint8_t)sb;
}

#ifndef QUANT_NT_BYTES
#define QUANT_NT_BYTES (128ll << 20)
#endif

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream, bool groups) {
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 511) / 512), (unsigned)((rows + 31) / 32));
  // Inputs above QUANT_NT_BYTES are read and their codes written with nontemporal
  // accesses: a tensor that size cannot stay in the 256 MB Infinity Cache for its
  // consumers anyway, and streaming it past the caches took the 419 MB X of a 32760 x
  // 5120 workload from 67.6 to 72.9% of 8 TB/s. Smaller inputs keep cached accesses,
  // which win when the tensor is still resident from its producer.
  const bool nt = rows * ld * (bf16 ? 2 : 4) > QUANT_NT_BYTES;
  auto go = [&](auto kernel, const auto* xp) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, xp, rows, cols, ld, codes, scales); };
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const float* xf = static_cast<const float*>(x);
  if (bf16 && groups) go(k_quantize<bf16_t, true, false>, xb);
  else if (bf16) nt ? go(k_quantize<bf16_t, false, true>, xb) : go(k_quantize<bf16_t, false, false>, xb);
  else if (groups) go(k_quantize<float, true, false>, xf);
  else nt ? go(k_quantize<float, false, true>, xf) : go(k_quantize<float, false, false>, xf);
  return hipGetLastError();
}

}  // namespace ft
