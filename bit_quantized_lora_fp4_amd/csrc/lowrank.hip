// Low-rank side of the backward pass (FourTune §3.2: gradients propagate through all
// three branches; parameter updates are computed for the adapter only).
//
// k_prep_bwd   : [B | L2]^T in workspace (the operand layout the G-side
//                down-projection reads), and zeroed tile counters for k_lora_grad.
// k_lora_grad  : dA = GB[:, :r]^T bf16(X) and dB = bf16(G)^T XL[:, :r], reductions over
//                the M rows on bf16 MFMA. Both operands are m-major in memory, so
//                64-row slabs are staged in LDS and read transposed with
//                ds_read_b64_tr_b16. HBM-bound: it re-reads X and G once.
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {


// ------------------------------------------------------------------ prep (transposes)
constexpr int TT = 64;  // transpose tile

// U [N x rt], U(n, j) = j < r ? B[n, j] : L2[n, j - r]  ->  Ut [rt x N]
__global__ __launch_bounds__(256) void k_prep_bwd(const PrepArgs a) {
  __shared__ bf16_t tile[TT][TT + 2];
  const int rt = a.r + a.s;
  const int64_t ntc = (rt + TT - 1) / TT;
  const int64_t tiles = ((a.N + TT - 1) / TT) * ntc;
  const int64_t b = blockIdx.x;
  if (b == 0)
    for (int i = threadIdx.x; i < a.ncounters; i += 256) a.counters[i] = 0u;
  if (b >= tiles) return;
  const int64_t r0 = (b / ntc) * TT, c0 = (b % ntc) * TT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < TT; i += 4) {
    const int64_t n = r0 + i, j = c0 + tx;
    bf16_t v = 0;
    if (n < a.N && j < rt) v = j < a.r ? a.B[n * a.r + j] : a.L2[n * a.s + (j - a.r)];
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < TT; i += 4) {
    const int64_t j = c0 + i, n = r0 + tx;
    if (j < rt && n < a.N) a.Ut[j * a.N + n] = tile[tx][i];
  }
}

// ------------------------------------------------------------------ LoRA gradients
// Output tile: RP (= r rounded up to 32) small rows x 256 big columns, one workgroup
// per (tile, M-split). 4 waves, each 64 big columns (2 MFMA column tiles).
constexpr int LG_BT = 256, LG_MS = 64;  // big-tile width, rows per LDS slab
constexpr int BIG_PITCH = LG_BT * 2 + 32;

// 8 consecutive elements of a bf16 or fp32 row as 8 bf16 (RNE for fp32).
__device__ __forceinline__ uint4 load8_bf16(const void* base, bool is_bf16, int64_t off, bool ok) {
  if (!ok) return make_uint4(0, 0, 0, 0);
  if (is_bf16) return *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(base) + off);
  const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
  const float4 a = p[0], b = p[1];
  return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                    pack_bf16x2(b.z, b.w));
}

template <int PT>  // small-side 32-row tiles (RP = 32 * PT)
__global__ __launch_bounds__(256) void k_lora_grad(const LoraGradArgs a) {
  constexpr int RP = 32 * PT;
  constexpr int SMALL_PITCH = RP * 2 + 32;
  __shared__ __align__(16) char s_big[LG_MS * BIG_PITCH];
  __shared__ __align__(16) char s_small[LG_MS * SMALL_PITCH];
  __shared__ uint32_t s_last;
  lds_char* big = (lds_char*)(s_big);
  lds_char* small = (lds_char*)(s_small);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tilesA = (int)((a.K + LG_BT - 1) / LG_BT);
  const int tile = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const bool jobA = tile < tilesA;
  // dA: small = GB (first r cols), big = X. dB^T: small = XL (first r cols), big = G.
  const bf16_t* sm = jobA ? a.gb : a.xl;
  const int64_t ld_sm = jobA ? a.ld_gb : a.ld_xl;
  const void* bg = jobA ? a.x : a.g;
  const bool bg_bf16 = jobA ? a.x_bf16 : a.g_bf16;
  const int64_t nbig = jobA ? a.K : a.N;
  const int64_t q0 = (int64_t)(jobA ? tile : tile - tilesA) * LG_BT;
  const int64_t per = ((a.M + a.splits - 1) / a.splits + LG_MS - 1) / LG_MS * LG_MS;
  const int64_t mb = split * per, me = min(a.M, mb + per);

  v16f acc[PT][2];
#pragma unroll
  for (int p = 0; p < PT; ++p) acc[p][0] = acc[p][1] = v16f{};

  for (int64_t m0 = mb; m0 < me; m0 += LG_MS) {
    // stage big slab [64 x 256] and small slab [64 x RP] as bf16
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 5, c8 = c & 31;
      const int64_t gm = m0 + row, gq = q0 + 8 * c8;
      const uint4 v = load8_bf16(bg, bg_bf16, gm * nbig + gq, gm < me && gq < nbig);
      *(__attribute__((address_space(3))) v4i*)(big + row * BIG_PITCH + c8 * 16) = __builtin_bit_cast(v4i, v);
    }
    for (int c = tid; c < LG_MS * (RP / 8); c += 256) {
      const int row = c / (RP / 8), c8 = c % (RP / 8);
      const int64_t gm = m0 + row;
      const bool ok = gm < me && 8 * c8 < a.r;
      const uint4 v = ok ? *reinterpret_cast<const uint4*>(sm + gm * ld_sm + 8 * c8) : make_uint4(0, 0, 0, 0);
      *(__attribute__((address_space(3))) v4i*)(small + row * SMALL_PITCH + c8 * 16) = __builtin_bit_cast(v4i, v);
    }
    __syncthreads();
#pragma unroll
    for (int ms = 0; ms < LG_MS; ms += 16) {
      v4i sa[PT], bb[2];
#pragma unroll
      for (int p = 0; p < PT; ++p) sa[p] = lds_tr16_pair(small, SMALL_PITCH, ms, 32 * p, lane);
#pragma unroll
      for (int q = 0; q < 2; ++q) bb[q] = lds_tr16_pair(big, BIG_PITCH, ms, wave * 64 + 32 * q, lane);
#pragma unroll
      for (int p = 0; p < PT; ++p)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sa[p]),
                                                             __builtin_bit_cast(bf16x8, bb[q]), acc[p][q], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- partials [splits][RP][K + N]: dA tiles at column q, dB^T tiles at column K + q
  const int64_t ptot = a.K + a.N;
  const int64_t pcol0 = (jobA ? 0 : a.K) + q0;
  auto out_final = [&](int p, int64_t q, float v) {
    if (p >= a.r || q >= nbig) return;
    if (jobA) a.dA[(int64_t)p * a.K + q] = v;
    else a.dB[q * a.r + p] = v;
  };
  if (a.splits == 1) {
#pragma unroll
    for (int p = 0; p < PT; ++p)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out_final(32 * p + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), q0 + wave * 64 + 32 * q + (lane & 31), acc[p][q][r]);
    return;
  }
  float* part = a.partials + (int64_t)split * RP * ptot;
#pragma unroll
  for (int p = 0; p < PT; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pr = 32 * p + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t qc = wave * 64 + 32 * q + (lane & 31);
        if (q0 + qc < nbig) part[(int64_t)pr * ptot + pcol0 + qc] = acc[p][q][r];
      }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.counters[tile], 1u) == (uint32_t)(a.splits - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // last split of this tile: fixed-order sum over splits
  const int width = (int)min((int64_t)LG_BT, nbig - q0);
  for (int e = tid; e < a.r * LG_BT; e += 256) {
    const int p = e / LG_BT, qc = e % LG_BT;
    if (qc >= width) continue;
    float s = 0.f;
    for (int sp = 0; sp < a.splits; ++sp)
      s += __builtin_nontemporal_load(a.partials + (int64_t)sp * RP * ptot + (int64_t)p * ptot + pcol0 + qc);
    out_final(p, q0 + qc, s);
  }
  if (tid == 0) a.counters[tile] = 0u;
}

}  // namespace

hipError_t launch_prep_bwd(const PrepArgs& a, hipStream_t stream) {
  const int rt = a.r + a.s;
  const int64_t tiles = ((a.N + TT - 1) / TT) * ((rt + TT - 1) / TT);
  const int64_t blocks = tiles > 0 ? tiles : 1;
  hipLaunchKernelGGL(k_prep_bwd, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int lora_grad_tiles(int64_t K, int64_t N) {
  return (int)((K + LG_BT - 1) / LG_BT + (N + LG_BT - 1) / LG_BT);
}

int lora_grad_splits(int64_t M, int64_t K, int64_t N) {
  const int tiles = lora_grad_tiles(K, N);
  int64_t s = 512 / tiles;
  s = s < 1 ? 1 : s;
  const int64_t maxs = (M + 255) / 256;  // at least 256 rows per split
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

hipError_t launch_lora_grad(const LoraGradArgs& a, hipStream_t stream) {
  if (a.r == 0 || a.M == 0) return hipSuccess;
  const int tiles = lora_grad_tiles(a.K, a.N);
  dim3 grid((unsigned)(tiles * a.splits)), block(256);
  switch ((a.r + 31) / 32) {
    case 1: hipLaunchKernelGGL(k_lora_grad<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(k_lora_grad<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_lora_grad<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(k_lora_grad<4>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ft
