// Fused quantization + low-rank down-projection (FourTune §3.3 "LoRA Fusion": all
// three branches read the same input, so its quantization and every down-projection
// happen in one kernel and the input is read from HBM once).
//
//   forward : X -> Q(X), XL = bf16( bf16(X) [A; L1]^T )          D = [A; L1]
//   backward: G -> Q(G), GB = bf16( bf16(G) [B | L2] )            D = [B | L2]^T
//
// HBM-bound: 2 (bf16) or 4 (fp32) bytes read and 0.5 written per element, plus the
// small [M x rt] output. The down-projection runs on bf16 MFMA (32x32x16) straight
// from the registers the quantizer loaded.
//
// Mapping. One workgroup of 8 waves owns a 32-row stripe; wave w walks the stripe's
// 128-column chunks w, w+8, ... with the next chunk's loads in flight while it works
// on the current one. Inside a chunk lane l holds row l%32 and, for each of the 8
// 16-column steps, the 8 columns (l/32)*8 .. +8 of the step: exactly the A operand of
// the bf16 MFMA, and for the quantizer each 32x32 block is two steps. Block maxima
// are combined over all 64 lanes with butterflies; the E2M1 conversion is the
// hardware one. The 8 waves' fp32 partial products meet in LDS and are summed in wave
// order before the single bf16 rounding.
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {

constexpr int QD_WAVES = 8;

template <typename T>
struct Chunk;

template <>
struct Chunk<bf16_t> {
  uint4 v[8];  // step s: 8 bf16 at columns c0 + 16s + 8*(l/32)
  __device__ void load(const bf16_t* row_ptr, int64_t c0, int64_t K, int half, bool row_ok) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t c = c0 + 16 * s + 8 * half;
      v[s] = (row_ok && c < K) ? *reinterpret_cast<const uint4*>(row_ptr + c) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ uint32_t absmax(int s) const {
    return umax(umax(bf16x2_absmax_bits(v[s].x), bf16x2_absmax_bits(v[s].y)),
                umax(bf16x2_absmax_bits(v[s].z), bf16x2_absmax_bits(v[s].w)));
  }
  __device__ uint32_t codes(int s, float scale) const { return cvt8_bf16(v[s].x, v[s].y, v[s].z, v[s].w, scale); }
  __device__ v4i operand(int s) const { return v4i{(int)v[s].x, (int)v[s].y, (int)v[s].z, (int)v[s].w}; }
};

template <>
struct Chunk<float> {
  float4 v[8][2];
  __device__ void load(const float* row_ptr, int64_t c0, int64_t K, int half, bool row_ok) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t c = c0 + 16 * s + 8 * half;
      const bool ok = row_ok && c < K;
      v[s][0] = ok ? reinterpret_cast<const float4*>(row_ptr + c)[0] : make_float4(0, 0, 0, 0);
      v[s][1] = ok ? reinterpret_cast<const float4*>(row_ptr + c)[1] : make_float4(0, 0, 0, 0);
    }
  }
  __device__ uint32_t absmax(int s) const {
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m = umax(m, __builtin_bit_cast(uint32_t, v[s][h].x) & 0x7FFFFFFFu);
      m = umax(m, __builtin_bit_cast(uint32_t, v[s][h].y) & 0x7FFFFFFFu);
      m = umax(m, __builtin_bit_cast(uint32_t, v[s][h].z) & 0x7FFFFFFFu);
      m = umax(m, __builtin_bit_cast(uint32_t, v[s][h].w) & 0x7FFFFFFFu);
    }
    return m;
  }
  __device__ uint32_t codes(int s, float scale) const {
    const float f[8] = {v[s][0].x, v[s][0].y, v[s][0].z, v[s][0].w,
                        v[s][1].x, v[s][1].y, v[s][1].z, v[s][1].w};
    return cvt8_f32(f, scale);
  }
  __device__ v4i operand(int s) const {  // bf16(x), round to nearest even
    return v4i{(int)pack_bf16x2(v[s][0].x, v[s][0].y), (int)pack_bf16x2(v[s][0].z, v[s][0].w),
               (int)pack_bf16x2(v[s][1].x, v[s][1].y), (int)pack_bf16x2(v[s][1].z, v[s][1].w)};
  }
};

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = umax(v, shfl_xor_u32<1>(v));
  v = umax(v, shfl_xor_u32<2>(v));
  v = umax(v, shfl_xor_u32<4>(v));
  v = umax(v, shfl_xor_u32<8>(v));
  v = umax(v, shfl_xor_u32<16>(v));
  v = umax(v, shfl_xor_u32<32>(v));
  return v;
}

template <typename T, int RT_TILES>
__global__ __launch_bounds__(512) void k_quant_down(const QuantDownArgs a) {
  __shared__ float red[QD_WAVES][RT_TILES > 0 ? RT_TILES : 1][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * 32;
  const int64_t row = r0 + (lane & 31);
  const bool row_ok = row < a.M;
  const T* xrow = static_cast<const T*>(a.x) + row * a.ldx;
  const int64_t nchunks = (a.K + 127) / 128;
  const int64_t cpitch = a.K >> 1, nkb = a.K >> 5;

  // D rows this lane feeds into the B operand: j = 32*jt + l%32
  const bf16_t* drow[RT_TILES > 0 ? RT_TILES : 1];
#pragma unroll
  for (int jt = 0; jt < RT_TILES; ++jt) {
    const int j = 32 * jt + (lane & 31);
    drow[jt] = j < a.r0 ? a.d0 + (int64_t)j * a.K : a.d1 + (int64_t)(j - a.r0) * a.K;
  }
  v16f acc[RT_TILES > 0 ? RT_TILES : 1];
#pragma unroll
  for (int jt = 0; jt < RT_TILES; ++jt) acc[jt] = v16f{};

  Chunk<T> cur, nxt;
  int64_t c = wave;
  if (c < nchunks) cur.load(xrow, c * 128, a.K, half, row_ok);
  for (; c < nchunks; c += QD_WAVES) {
    const int64_t c0 = c * 128;
    if (c + QD_WAVES < nchunks) nxt.load(xrow, (c + QD_WAVES) * 128, a.K, half, row_ok);

    // ---- quantize the chunk's (up to) four 32x32 blocks
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t bc = c0 + 32 * b;
      if (bc >= a.K) break;  // uniform
      const uint32_t amax = wave_max(umax(cur.absmax(2 * b), cur.absmax(2 * b + 1)));
      const uint32_t sb = scale_byte_from_amax(amax);
      const float scale = e8m0_to_f32_scale(sb);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t cw = cur.codes(2 * b + h, scale);
        if (sb == 0xFFu) cw = 0;
        if (row_ok)
          *reinterpret_cast<uint32_t*>(a.codes + row * cpitch + ((bc + 16 * h + 8 * half) >> 1)) = cw;
      }
      if (lane == 0) a.scales[blockIdx.x * nkb + (bc >> 5)] = (uint8_t)sb;
    }
    // ---- down-projection on bf16 MFMA
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t kc = c0 + 16 * s + 8 * half;
      const v4i xa = cur.operand(s);
#pragma unroll
      for (int jt = 0; jt < RT_TILES; ++jt) {
        const v4i db = kc < a.K ? *reinterpret_cast<const v4i*>(drow[jt] + kc) : v4i{0, 0, 0, 0};
        acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa),
                                                          __builtin_bit_cast(bf16x8, db), acc[jt], 0, 0, 0);
      }
    }
    cur = nxt;
  }

  if constexpr (RT_TILES > 0) {
#pragma unroll
    for (int jt = 0; jt < RT_TILES; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][jt][r][lane] = acc[jt][r];
    __syncthreads();
    // 32 rows x rt outputs; thread t sums the 8 waves' partials in order
    const int total = 32 * 32 * RT_TILES;
    for (int e = threadIdx.x; e < total; e += 512) {
      const int jt = e / 1024, rem = e % 1024;
      const int r = rem / 64, l = rem % 64;  // accumulator element (register r, lane l)
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < QD_WAVES; ++w) s += red[w][jt][r][l];
      const int64_t orow = r0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const int ocol = 32 * jt + (l & 31);
      if (orow < a.M) a.low[orow * a.rt + ocol] = (bf16_t)f32_to_bf16_bits(s);
    }
  }
}

template <typename T>
hipError_t launch_t(const QuantDownArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + 31) / 32)), block(512);
  switch (a.rt / 32) {
    case 0: hipLaunchKernelGGL((k_quant_down<T, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((k_quant_down<T, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_quant_down<T, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((k_quant_down<T, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_quant_down<T, 4>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_down(const QuantDownArgs& a, bool x_bf16, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  return x_bf16 ? launch_t<bf16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace ft
