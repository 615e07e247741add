// LoRA parameter gradients (FourTune §3.2: gradients flow through all three branches,
// only the adapter is updated):
//
//   dA [r x K] = GB[:, :r]^T bf16(X)          dB [N x r] = bf16(G)^T XL[:, :r]
//
// Both are reductions over the M token rows of a narrow "small" operand (GB or XL,
// bf16 [M x rt]) against a wide "big" one (X or G, bf16 or fp32). HBM-bound: X and G
// are read once more, everything else is small; the flops run on bf16 MFMA.
//
// Work split. The output is cut into tiles of RP (r rounded up to 32) x Q (64 or 128) big
// columns; the dA tiles come first, then the dB tiles. A workgroup owns one tile and
// one of S contiguous 32-aligned row ranges; its 4 waves take the range's 32-row slabs
// in turn (w, w+4, ...), each with the next slab's loads in flight. Both operands are
// row-major in m, but the MFMA reduces over m inside a lane, so a wave writes its slab
// into a private LDS area and reads it back transposed (ds_read_b64_tr_b16). At the
// end the four waves' sums meet in LDS in wave order; with S > 1 the range sums go to
// an fp32 partial buffer and the S partials are added in range order afterwards, by
// k_lora_reduce or by extra workgroups of the backward GEMM's launch (LoraReduce). The
// result is independent of timing.
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {

constexpr int LG_WAVES = 4;
constexpr int LG_SLAB = 32;    // rows per wave slab

// Big columns per tile: 64, or 128 from 8192 rows up to rank 64 (with rank > 64 the
// waves' [RP x 128] fp32 sums would not fit the LDS). The wider tile reads 256
// contiguous bytes of each big row instead of 128 and the small operand half as often:
// at 9216 x 3072 x 9216, rank 64, the kernel went from 68.8 to 52.9 us (plus a 5 us
// reduction). At 4608 x 3072 x 3072, rank 32, it ran 17.5 -> 15.5 us as well, but the
// whole fused linear, called back to back, got slower (0.1169-0.1179 -> 0.1196-0.1204 ms
// per forward + backward), so shorter inputs keep 64.
int lg_q_for(int64_t M, int r) { return M >= 8192 && (r + 31) / 32 <= 2 ? 128 : 64; }

template <bool BIG_BF16, int PT, int Q>
struct Slab {
  static constexpr int RP = 32 * PT;
  static constexpr int UB = Q / 8;             // 16-byte units of a big row
  static constexpr int BIG_PITCH = Q * 2 + 16;
  static constexpr int NB = BIG_BF16 ? Q / 16 : Q / 8;  // 16-byte big loads per lane
  static constexpr int NS = RP / 16;           // 16-byte small loads per lane
  v4i big[NB];
  v4i small[NS];

  // big: unit e = i*64 + lane -> row e/UB, 8 columns at 8*(e%UB)
  // small: unit e = i*64 + lane -> row e/(RP/8), 8 columns at 8*(e%(RP/8))
  __device__ void load(bufres rb, bufres rs, int64_t m0, int64_t q0, int64_t nbig, int64_t ld_big,
                       int64_t ld_small, int r, int lane) {
#pragma unroll
    for (int i = 0; i < Q / 16; ++i) {
      const int e = i * 64 + lane, row = e / UB;
      const int64_t q = q0 + 8 * (e % UB);
      const int64_t m = m0 + row;
      const bool ok = q < nbig;
      if constexpr (BIG_BF16) {
        big[i] = buf_load16(rb, sel_off(ok, (uint32_t)((m * ld_big + q) * 2)));
      } else {
        const uint32_t off = sel_off(ok, (uint32_t)((m * ld_big + q) * 4));
        big[2 * i] = buf_load16(rb, off);
        big[2 * i + 1] = buf_load16(rb, off + 16);  // OOB + 16 is still OOB
      }
    }
    constexpr int UPR = RP / 8;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = i * 64 + lane, row = e / UPR, p = 8 * (e % UPR);
      const int64_t m = m0 + row;
      small[i] = buf_load16(rs, sel_off(p < r, (uint32_t)((m * ld_small + p) * 2)));
    }
  }

  __device__ void stage(lds_char* sbig, lds_char* ssmall, int small_pitch, int lane, bool gelu) const {
#pragma unroll
    for (int i = 0; i < Q / 16; ++i) {
      const int e = i * 64 + lane;
      v4i v;
      if constexpr (BIG_BF16) {
        v = big[i];
        if (gelu)  // uniform: bf16(GELU(P^)) for the MLP's second linear
          v = v4i{(int)gelu_bf16x2((uint32_t)v.x), (int)gelu_bf16x2((uint32_t)v.y),
                  (int)gelu_bf16x2((uint32_t)v.z), (int)gelu_bf16x2((uint32_t)v.w)};
      } else {
        const v4f a = __builtin_bit_cast(v4f, big[2 * i]), b = __builtin_bit_cast(v4f, big[2 * i + 1]);
        v = v4i{(int)pack_bf16x2(a.x, a.y), (int)pack_bf16x2(a.z, a.w), (int)pack_bf16x2(b.x, b.y),
                (int)pack_bf16x2(b.z, b.w)};
      }
      *(__attribute__((address_space(3))) v4i*)(sbig + (e / UB) * BIG_PITCH + (e % UB) * 16) = v;
    }
    constexpr int UPR = RP / 8;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = i * 64 + lane;
      *(__attribute__((address_space(3))) v4i*)(ssmall + (e / UPR) * small_pitch + (e % UPR) * 16) = small[i];
    }
  }
};

template <bool BIG_BF16, int PT, int LG_Q>
__global__ __launch_bounds__(256) void k_lora_grad(const LoraGradArgs a) {
  constexpr int RP = 32 * PT;
  constexpr int NQ = LG_Q / 32;
  using Sl = Slab<BIG_BF16, PT, LG_Q>;
  constexpr int BIG_PITCH = Sl::BIG_PITCH;
  constexpr int SMALL_PITCH = RP * 2 + 16;
  constexpr int STAGE = LG_SLAB * BIG_PITCH + LG_SLAB * SMALL_PITCH;  // per wave
  constexpr int RED = LG_WAVES * RP * LG_Q * 4;
  constexpr int SMEM = LG_WAVES * STAGE > RED ? LG_WAVES * STAGE : RED;
  __shared__ __align__(16) char smem_raw[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = gridDim.y, split = blockIdx.y;
  const int tilesA = (int)((a.K + LG_Q - 1) / LG_Q);
  const int tile = blockIdx.x + a.tile_offset;
  const bool jobA = tile < tilesA;
  const bf16_t* sm = jobA ? a.gb : a.xl;
  const int64_t ld_sm = jobA ? a.ld_gb : a.ld_xl;
  const void* bg = jobA ? a.x : a.g;
  const int64_t nbig = jobA ? a.K : a.N;
  const int64_t q0 = (int64_t)(jobA ? tile : tile - tilesA) * LG_Q;
  const bool gelu = BIG_BF16 && a.gelu_x && jobA;
  const int64_t per = ((a.M + S - 1) / S + LG_SLAB - 1) / LG_SLAB * LG_SLAB;
  const int64_t mb = split * per, me = min(a.M, mb + per);

  const bufres rb = make_buf(bg, (uint64_t)a.M * nbig * (BIG_BF16 ? 2 : 4));
  const bufres rs = make_buf(sm, (uint64_t)a.M * ld_sm * 2);
  lds_char* sbig = (lds_char*)smem_raw + wave * STAGE;
  lds_char* ssmall = sbig + LG_SLAB * BIG_PITCH;

  v16f acc[PT][NQ];
#pragma unroll
  for (int p = 0; p < PT; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[p][q] = v16f{};

  // Two register sets in turn: one slab's loads are in flight while the other is
  // staged and multiplied. A slab past the range loads nothing (its row start is M,
  // beyond the buffers).
  auto load = [&](Sl& sl, int64_t m0) {
    sl.load(rb, rs, m0 < me ? m0 : a.M, q0, nbig, nbig, ld_sm, a.r, lane);
  };
  auto work = [&](const Sl& sl) {
    sl.stage(sbig, ssmall, SMALL_PITCH, lane, gelu);
#pragma unroll
    for (int ms = 0; ms < LG_SLAB; ms += 16) {
      v4i sa[PT], bb[NQ];
#pragma unroll
      for (int p = 0; p < PT; ++p) sa[p] = lds_tr16_pair(ssmall, SMALL_PITCH, ms, 32 * p, lane);
#pragma unroll
      for (int q = 0; q < NQ; ++q) bb[q] = lds_tr16_pair(sbig, BIG_PITCH, ms, 32 * q, lane);
#pragma unroll
      for (int p = 0; p < PT; ++p)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sa[p]),
                                                             __builtin_bit_cast(bf16x8, bb[q]), acc[p][q], 0, 0, 0);
    }
  };
  // Two slabs per trip, each in its own register set; the second may lie past the
  // range (it then loads zeros), which keeps the trip branch-free. Scheduling barriers
  // keep each half's arithmetic after the loads of the other half are issued.
  constexpr int STEP = LG_WAVES * LG_SLAB;
  Sl s0, s1;
  int64_t m0 = mb + (int64_t)wave * LG_SLAB;
  load(s0, m0);
  for (; m0 < me; m0 += 2 * STEP) {
    load(s1, m0 + STEP);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    work(s0);
    __builtin_amdgcn_sched_barrier(0);
    load(s0, m0 + 2 * STEP);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    work(s1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Rows past M were read as zero (buffer bounds), so the ragged last slab needs no mask.

  // ---- wave sums into LDS, [wave][p][q] fp32
  __syncthreads();
  float* red = (float*)smem_raw;
#pragma unroll
  for (int p = 0; p < PT; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pr = 32 * p + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        red[(wave * RP + pr) * LG_Q + 32 * q + (lane & 31)] = acc[p][q][r];
      }
  __syncthreads();

  // Tile element order matches the output's: dA rows p with q contiguous (index p*64+q),
  // dB rows q with p contiguous (index q*RP+p). Thread t handles 4 consecutive indices.
  const int width = (int)min((int64_t)LG_Q, nbig - q0);
  auto elem = [&](int idx, int& p, int& q) {
    if (jobA) { p = idx / LG_Q; q = idx % LG_Q; }
    else { q = idx / RP; p = idx % RP; }
  };
  auto store_final = [&](int idx, v4f v) {
    int p, q;
    elem(idx, p, q);
    if (p >= a.r || q >= width) return;
    if (jobA) {
      *reinterpret_cast<v4f*>(a.dA + (int64_t)p * a.K + q0 + q) = v;
    } else {
      *reinterpret_cast<v4f*>(a.dB + (q0 + q) * a.r + p) = v;
    }
  };
  constexpr int NE = RP * LG_Q;
  v4f sums[NE / 1024 > 0 ? NE / 1024 : 1];
#pragma unroll
  for (int i = 0; i < NE / 1024; ++i) {
    const int idx = 4 * (tid + 256 * i);
    int p, q;
    elem(idx, p, q);
    v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < LG_WAVES; ++w) {
      if (jobA) {
        s += *reinterpret_cast<const v4f*>(red + (w * RP + p) * LG_Q + q);
      } else {
        s.x += red[(w * RP + p + 0) * LG_Q + q];
        s.y += red[(w * RP + p + 1) * LG_Q + q];
        s.z += red[(w * RP + p + 2) * LG_Q + q];
        s.w += red[(w * RP + p + 3) * LG_Q + q];
      }
    }
    sums[i] = s;
  }
  if (S == 1) {
#pragma unroll
    for (int i = 0; i < NE / 1024; ++i) store_final(4 * (tid + 256 * i), sums[i]);
    return;
  }
  v4f* part = reinterpret_cast<v4f*>(a.partials);
#pragma unroll
  for (int i = 0; i < NE / 1024; ++i) part[((int64_t)split * a.ntiles + tile) * (NE / 4) + tid + 256 * i] = sums[i];
}

// Sum of the S row-range partials of every tile, in range order (same element order
// as k_lora_grad's tiles), written to dA / dB.
__global__ __launch_bounds__(256) void k_lora_reduce(const LoraReduce t) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < t.items) lora_reduce_item(t, i);
}

template <bool BIG_BF16>
hipError_t launch_t(const LoraGradArgs& a, int q, dim3 grid, hipStream_t stream) {
  const int pt = (a.r + 31) / 32;  // 32-wide rank tiles
  if (q == 128) {
    switch (pt) {
      case 1: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 1, 128>), grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 2, 128>), grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (pt) {
      case 1: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 1, 64>), grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 2, 64>), grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 3, 64>), grid, dim3(256), 0, stream, a); break;
      case 4: hipLaunchKernelGGL((k_lora_grad<BIG_BF16, 4, 64>), grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

int lora_grad_tiles(int64_t M, int64_t K, int64_t N, int r) {
  const int q = lg_q_for(M, r);
  return (int)((K + q - 1) / q + (N + q - 1) / q);
}

// Row ranges per tile: enough for about 192 workgroups while they fit one round of the
// 256 CUs. Fewer ranges mean fewer fp32 partials (written here, read again by
// k_lora_reduce) and longer-lived waves; at 4608 x 3072 (64-column tiles, 96 of them) 2
// ranges ran the fused linear ~1.5% faster than 6 (a 512 target), and 1 range was
// slower. Past one round the CUs end unevenly loaded (at 32760 rows with 64-column
// tiles, one range for each of 320 tiles: 441 us, the CUs holding two workgroups
// finishing last), and about 1024 workgroups even that out (315 us + 6.6 us of
// reduction there; with 128-column tiles, 160 x 7 ranges: 296 + 8.4 us against 327 +
// 5.3 us for 160 x 2).
constexpr int LG_TARGET_WGS = 192;
constexpr int LG_TARGET_WGS_WIDE = 1024;

int lora_grad_splits(int64_t M, int64_t K, int64_t N, int r) {
  const int tiles = lora_grad_tiles(M, K, N, r);
  int64_t s = (LG_TARGET_WGS + tiles - 1) / tiles;
  if (tiles * s > 256) s = (LG_TARGET_WGS_WIDE + tiles - 1) / tiles;
  const int64_t maxs = M / (2 * LG_WAVES * LG_SLAB);  // at least two slabs per wave
  if (s > maxs) s = maxs;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

size_t lora_grad_partial_bytes(int64_t M, int64_t K, int64_t N, int r) {
  const int S = lora_grad_splits(M, K, N, r);
  if (S <= 1 || r == 0) return 0;
  const int64_t rp = (r + 31) / 32 * 32;
  return (size_t)S * lora_grad_tiles(M, K, N, r) * rp * lg_q_for(M, r) * 4;
}

// Zero fill (the LoRA gradients of an empty batch): a kernel, not a memset node, so the
// call stays safe to capture in a graph.
__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const LoraGradArgs& a, hipStream_t stream, LoraReduce* deferred) {
  if (deferred) *deferred = LoraReduce{};
  if (a.r == 0 || a.M == 0) return hipSuccess;
  const int S = lora_grad_splits(a.M, a.K, a.N, a.r);
  const int LG_Q = lg_q_for(a.M, a.r);
  if (S > 1 && a.partials == nullptr) return hipErrorInvalidValue;
  const int tilesA = (int)((a.K + LG_Q - 1) / LG_Q), tiles = lora_grad_tiles(a.M, a.K, a.N, a.r);
  LoraGradArgs b = a;
  b.ntiles = tiles;
  hipError_t e;
  if (a.x_bf16 == a.g_bf16) {  // one launch for both jobs
    b.tile_offset = 0;
    e = a.x_bf16 ? launch_t<true>(b, LG_Q, dim3((unsigned)tiles, (unsigned)S), stream)
                 : launch_t<false>(b, LG_Q, dim3((unsigned)tiles, (unsigned)S), stream);
  } else {  // X and G differ in dtype: the dA tiles and the dB tiles are two launches
    b.tile_offset = 0;
    e = a.x_bf16 ? launch_t<true>(b, LG_Q, dim3((unsigned)tilesA, (unsigned)S), stream)
                 : launch_t<false>(b, LG_Q, dim3((unsigned)tilesA, (unsigned)S), stream);
    if (e != hipSuccess) return e;
    b.tile_offset = tilesA;
    e = a.g_bf16 ? launch_t<true>(b, LG_Q, dim3((unsigned)(tiles - tilesA), (unsigned)S), stream)
                 : launch_t<false>(b, LG_Q, dim3((unsigned)(tiles - tilesA), (unsigned)S), stream);
  }
  if (e != hipSuccess || S == 1) return e;
  LoraReduce t{};
  t.partials = a.partials;
  t.dA = a.dA;
  t.dB = a.dB;
  t.K = a.K;
  t.N = a.N;
  t.r = a.r;
  t.S = S;
  t.rp = (a.r + 31) / 32 * 32;
  t.q = LG_Q;
  t.ntiles = tiles;
  t.items = (int64_t)tiles * t.rp * LG_Q / 4;
  if (deferred) {
    *deferred = t;
    return hipSuccess;
  }
  hipLaunchKernelGGL(k_lora_reduce, dim3((unsigned)((t.items + 255) / 256)), dim3(256), 0, stream, t);
  return hipGetLastError();
}

}  // namespace ft
