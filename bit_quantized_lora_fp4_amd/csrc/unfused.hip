// Unfused building blocks, used only to measure what the fusions save (FourTune §4,
// "Kernel Fusion Breakdown", Figure 9): the low-rank up-projection added to a backbone
// product that was stored in HBM, and GELU / GELU' as separate elementwise passes.
// The fused path never calls these.
#include "common.h"
#include "gemm.h"
#include "launch.h"

namespace ft {

namespace {

constexpr int UA_ROWS = 128;               // output rows per workgroup (32 per wave)
constexpr int UA_COLS = 128;               // output columns per workgroup (4 MFMA tiles)
constexpr int UA_THREADS = 256;
constexpr int UT_PITCH_BWD = UA_COLS * 2 + 32;  // staged D row: 128 bf16 + 32 bytes (tr16 banks)
constexpr int ST_COLS = 64;                // output columns staged per pass (two passes)
constexpr int ST_PITCH = ST_COLS * 4 + 16;  // staged fp32 output row
constexpr int ST_WAVE = 32 * ST_PITCH;
constexpr int UA_LDS = (128 * UT_PITCH_BWD > 4 * ST_WAVE) ? 128 * UT_PITCH_BWD : 4 * ST_WAVE;

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// out[M x C] = base[M x C] + low[M x rt] * V, fp32 accumulation, one rounding.
//   forward : V = U^T, U [C x rt] = [B | L2] (row q of U is v0 row q ++ v1 row q)
//   backward: V = D,   D [rt x C] = [A; L1]  (row j of D is v0 row j, or v1 row j - r0)
// The workgroup stages its 128 columns of V in LDS (forward: as [column][rank], read
// with 16-byte reads; backward: as [rank][column], read transposed with
// ds_read_b64_tr_b16), each wave takes 32 rows. The MFMA runs with V as the first
// operand, so a lane's accumulator holds four consecutive columns of one row; the
// result goes through LDS once more so that base is read and out written as 128
// contiguous bytes per row and pass.
template <bool BWD, bool OUT_BF16>
__global__ __launch_bounds__(UA_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void k_up_add(UpAddArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_raw[UA_LDS];
  lds_char* const lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t M = a.M, C = a.C;
  const int rt = a.rt, r0 = a.r0;
  const int64_t c0 = (int64_t)blockIdx.x * UA_COLS;
  const int64_t m0 = (int64_t)blockIdx.y * UA_ROWS + 32 * wave;

  // base rows this lane adds, prefetched: pass h, slot i -> row m0 + 8i + lane/8,
  // columns c0 + 64h + 8(lane%8) .. +8
  const bufres bb = make_buf(a.base, (uint64_t)M * C * 2);
  v4i base_v[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + 8 * i + (lane >> 3), col = c0 + ST_COLS * h + 8 * (lane & 7);
      base_v[h][i] = buf_load16(bb, sel_off(row < M && col < C, (uint32_t)((row * C + col) * 2)));
    }

  // low operand (second MFMA operand): row m0 + lane%32, ranks 16kk + 8(lane/32) .. +8
  const bufres bl = make_buf(a.low, (uint64_t)M * rt * 2);
  v4i lo[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    if (16 * kk < rt)
      lo[kk] = buf_load16(bl, (uint32_t)(((m0 + (lane & 31)) * rt + 16 * kk + 8 * (lane >> 5)) * 2));

  // stage V's 128 columns
  const int s1 = rt - r0;
  const bufres b0 = make_buf(a.v0, BWD ? (uint64_t)r0 * C * 2 : (uint64_t)C * r0 * 2);
  const bufres b1 = make_buf(a.v1, BWD ? (uint64_t)s1 * C * 2 : (uint64_t)C * s1 * 2);
  if constexpr (!BWD) {
    const int pitch = rt * 2 + 16;
    const int per_row = rt / 8;  // 16-byte pieces per staged row
    for (int q = tid; q < UA_COLS * per_row; q += UA_THREADS) {
      const int c = q / per_row, k = 8 * (q % per_row);
      const int64_t col = c0 + c;
      v4i v;
      if (k < r0)
        v = buf_load16(b0, sel_off(col < C, (uint32_t)((col * r0 + k) * 2)));
      else
        v = buf_load16(b1, sel_off(col < C, (uint32_t)((col * s1 + k - r0) * 2)));
      *(__attribute__((address_space(3))) v4i*)(lds + c * pitch + 2 * k) = v;
    }
  } else {
    for (int q = tid; q < rt * (UA_COLS / 8); q += UA_THREADS) {
      const int k = q / (UA_COLS / 8), c = 8 * (q % (UA_COLS / 8));
      const int64_t col = c0 + c;
      v4i v;
      if (k < r0)
        v = buf_load16(b0, sel_off(col < C, (uint32_t)(((int64_t)k * C + col) * 2)));
      else
        v = buf_load16(b1, sel_off(col < C, (uint32_t)(((int64_t)(k - r0) * C + col) * 2)));
      *(__attribute__((address_space(3))) v4i*)(lds + k * UT_PITCH_BWD + 2 * c) = v;
    }
  }
  __syncthreads();

  v16f acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (16 * kk >= rt) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4i v;
      if constexpr (!BWD)
        v = *(const __attribute__((address_space(3))) v4i*)(lds + (32 * j + (lane & 31)) * (rt * 2 + 16) +
                                                             2 * (16 * kk + 8 * (lane >> 5)));
      else
        v = lds_tr16_pair(lds, UT_PITCH_BWD, 16 * kk, 32 * j, lane);
      acc[j] = mfma_bf16(v, lo[kk], acc[j]);
    }
  }
  __syncthreads();  // V no longer read: its LDS now stages the output

  // acc[j][r] is out[m0 + lane%32][c0 + 32j + 8(r/4) + 4(lane/32) + r%4]
  lds_char* const stw = lds + wave * ST_WAVE;
  const bufres bo = make_buf(a.out, (uint64_t)M * C * (OUT_BF16 ? 2 : 4));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v16f& t = acc[2 * h + jj];
        v4f w = {t[4 * g], t[4 * g + 1], t[4 * g + 2], t[4 * g + 3]};
        *(__attribute__((address_space(3))) v4f*)(stw + (lane & 31) * ST_PITCH +
                                                  4 * (32 * jj + 8 * g + 4 * (lane >> 5))) = w;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 8 * i + (lane >> 3), cl = 8 * (lane & 7);
      const lds_char* p = stw + rl * ST_PITCH + 4 * cl;
      const v4f x0 = *(const __attribute__((address_space(3))) v4f*)p;
      const v4f x1 = *(const __attribute__((address_space(3))) v4f*)(p + 16);
      const v4i bv = base_v[h][i];
      float s[8] = {x0[0] + bf16_lo(bv.x), x0[1] + bf16_hi(bv.x), x0[2] + bf16_lo(bv.y), x0[3] + bf16_hi(bv.y),
                    x1[0] + bf16_lo(bv.z), x1[1] + bf16_hi(bv.z), x1[2] + bf16_lo(bv.w), x1[3] + bf16_hi(bv.w)};
      const int64_t row = m0 + rl, col = c0 + ST_COLS * h + cl;
      const bool ok = row < M && col < C;
      if constexpr (OUT_BF16) {
        v4i o;
        o.x = (int)pack_bf16x2(s[0], s[1]);
        o.y = (int)pack_bf16x2(s[2], s[3]);
        o.z = (int)pack_bf16x2(s[4], s[5]);
        o.w = (int)pack_bf16x2(s[6], s[7]);
        if (ok) __builtin_amdgcn_raw_buffer_store_b128(o, bo, (int)((row * C + col) * 2), 0, 0);
      } else {
        v4i o0 = {__builtin_bit_cast(int, s[0]), __builtin_bit_cast(int, s[1]), __builtin_bit_cast(int, s[2]),
                  __builtin_bit_cast(int, s[3])};
        v4i o1 = {__builtin_bit_cast(int, s[4]), __builtin_bit_cast(int, s[5]), __builtin_bit_cast(int, s[6]),
                  __builtin_bit_cast(int, s[7])};
        if (ok) {
          __builtin_amdgcn_raw_buffer_store_b128(o0, bo, (int)((row * C + col) * 4), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(o1, bo, (int)((row * C + col) * 4 + 16), 0, 0);
        }
      }
    }
    __syncthreads();
  }
}

// h = bf16(GELU(p)) and dp = bf16(dh * GELU'(p)), 8 bf16 per lane per step. GELU and
// its derivative are the same fp32 functions the fused GEMM epilogues evaluate.
__global__ __launch_bounds__(256) void k_gelu(const bf16_t* p, bf16_t* h, int64_t n8) {
  const v4i* pv = reinterpret_cast<const v4i*>(p);
  v4i* hv = reinterpret_cast<v4i*>(h);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const v4i x = __builtin_nontemporal_load(pv + i);
    v4i y;
    y.x = (int)gelu_bf16x2((uint32_t)x.x);
    y.y = (int)gelu_bf16x2((uint32_t)x.y);
    y.z = (int)gelu_bf16x2((uint32_t)x.z);
    y.w = (int)gelu_bf16x2((uint32_t)x.w);
    __builtin_nontemporal_store(y, hv + i);
  }
}

__device__ __forceinline__ uint32_t dgelu_bf16x2(uint32_t dh, uint32_t p) {
  return pack_bf16x2(bf16_lo(dh) * gelu_grad_f(bf16_lo(p)), bf16_hi(dh) * gelu_grad_f(bf16_hi(p)));
}

__global__ __launch_bounds__(256) void k_gelu_bwd(const bf16_t* p, const bf16_t* dh, bf16_t* dp, int64_t n8) {
  const v4i* pv = reinterpret_cast<const v4i*>(p);
  const v4i* gv = reinterpret_cast<const v4i*>(dh);
  v4i* ov = reinterpret_cast<v4i*>(dp);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const v4i x = __builtin_nontemporal_load(pv + i);
    const v4i g = __builtin_nontemporal_load(gv + i);
    v4i y;
    y.x = (int)dgelu_bf16x2((uint32_t)g.x, (uint32_t)x.x);
    y.y = (int)dgelu_bf16x2((uint32_t)g.y, (uint32_t)x.y);
    y.z = (int)dgelu_bf16x2((uint32_t)g.z, (uint32_t)x.z);
    y.w = (int)dgelu_bf16x2((uint32_t)g.w, (uint32_t)x.w);
    __builtin_nontemporal_store(y, ov + i);
  }
}

int elementwise_grid(int64_t n8) {
  const int64_t per = 256 * 4;  // four 16-byte vectors per thread per launch-wide pass
  int64_t g = (n8 + per - 1) / per;
  if (g > 4096) g = 4096;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_up_add(const UpAddArgs& a, bool bwd, bool out_bf16, hipStream_t stream) {
  if (a.M == 0 || a.C == 0) return hipSuccess;
  if (a.rt <= 0 || a.rt % 16 != 0 || a.rt > 128 || a.r0 % 16 != 0 || a.r0 < 0 || a.r0 > a.rt || a.C % 8 != 0)
    return hipErrorInvalidValue;
  // 32-bit buffer offsets
  if ((uint64_t)a.M * a.C * (out_bf16 ? 2 : 4) >= 0xFFFFFF00ull || (uint64_t)(a.M + UA_ROWS) * a.rt * 2 >= 0xFFFFFF00ull)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.C + UA_COLS - 1) / UA_COLS), (unsigned)((a.M + UA_ROWS - 1) / UA_ROWS));
  if (grid.y > 65535u) return hipErrorInvalidValue;
  if (bwd && out_bf16)
    hipLaunchKernelGGL((k_up_add<true, true>), grid, dim3(UA_THREADS), 0, stream, a);
  else if (bwd)
    hipLaunchKernelGGL((k_up_add<true, false>), grid, dim3(UA_THREADS), 0, stream, a);
  else if (out_bf16)
    hipLaunchKernelGGL((k_up_add<false, true>), grid, dim3(UA_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((k_up_add<false, false>), grid, dim3(UA_THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gelu(const bf16_t* p, bf16_t* h, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (n % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gelu, dim3(elementwise_grid(n / 8)), dim3(256), 0, stream, p, h, n / 8);
  return hipGetLastError();
}

hipError_t launch_gelu_bwd(const bf16_t* p, const bf16_t* dh, bf16_t* dp, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (n % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gelu_bwd, dim3(elementwise_grid(n / 8)), dim3(256), 0, stream, p, dh, dp, n / 8);
  return hipGetLastError();
}

}  // namespace ft
