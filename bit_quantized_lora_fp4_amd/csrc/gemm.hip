// 4-bit backbone GEMMs of the W4A4G4 linear on gfx950 scaled-FP4 MFMA, with the
// low-rank up-projection accumulated into the same accumulators (FourTune §3.3 "LoRA
// Fusion": the 4-bit backbone is fused with the up-projections so the branch outputs
// are summed before one store).
//
//   forward  (TRANS_B = false): Y  = deq Q(X) deq Q(R)^T + XL [B|L2]^T     (§3.1)
//   backward (TRANS_B = true ): dX = deq Q(G) deq Q(R)   + GB [A;L1]       (§3.2)
//
// Operand A is always an MXFP4 tensor [M x Kred] read along its rows. Operand B is the
// frozen Q(R) [N x K]: the forward reads its rows (reduction over K); the backward
// reduces over N, i.e. reads Q(R) down its columns. Because the 32x32 block scales are
// local to a block, the backward uses the very same codes and scale bytes: code tiles
// are staged row-major in LDS and read transposed with ds_read_b64_tr_b4 (a 16x16
// nibble transpose across 16 lanes), and each lane picks the scale byte of the block
// its 32 reduction elements fall in (§3.2: a 4-bit block and its scale are fetched
// together in either orientation, with no dequantize/requantize).
//
// Tiling. A workgroup of 4 waves computes a 256 x 256 output tile; each wave a
// 128 x 128 quarter as 4 x 4 tiles of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP4 x FP4,
// E8M0 scale per lane = per 32 reduction elements). The reduction advances 128
// elements per step; each step's A and B code tiles (16 KB each) are double-buffered
// in LDS, the next step's global loads being in flight while the current step's 32
// MFMAs per wave run. LDS rows are XOR-swizzled in 16-byte units so that both the
// fragment reads and the staging writes are free of bank conflicts.
//
// MFMA operand layout (32x32x64, FP4): lane l holds row l%32 of its operand and the
// 32 reduction elements (l/32)*32 .. +32 of the 64-step, two per byte, even element
// in the low nibble; its scale operand byte (selected by op_sel) scales those 32.
// Accumulator register r of lane l is element (8*(r/4) + 4*(l/32) + r%4, l%32).
// The bf16 MFMA 32x32x16 uses the same accumulator layout, 8 bf16 per lane at
// reduction offset (l/32)*8.
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;  // output tile, reduction step (elements)
constexpr int WAVES = 4;
constexpr int TI = 4, TJ = 4;                 // 32x32 MFMA tiles per wave (rows, cols)
constexpr int A_TILE_BYTES = BM * BK / 2;     // 16 KB
constexpr int B_TILE_BYTES = BN * BK / 2;     // 16 KB

typedef __attribute__((address_space(3))) char lds_char;
typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i lds_read_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(p);
}
__device__ __forceinline__ void lds_write_b128(lds_char* p, v4i v) {
  *reinterpret_cast<__attribute__((address_space(3))) v4i*>(p) = v;
}
__device__ __forceinline__ v2i lds_read_tr4(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) v2i*)(p));
}

// A / forward-B tiles: 256 rows x 64 bytes, 16-byte unit c stored at unit c ^ ((row>>2)&3).
__device__ __forceinline__ int swz64(int row, int c16) {
  return row * 64 + ((c16 ^ ((row >> 2) & 3)) << 4);
}
// backward-B tile: 128 rows (reduction) x 128 bytes (256 output columns),
// 16-byte unit c stored at unit c ^ ((row>>1)&7).
__device__ __forceinline__ int swz128(int row, int c16) {
  return row * 128 + ((c16 ^ ((row >> 1) & 7)) << 4);
}

struct Frag {  // global -> LDS staging registers of one thread for one operand tile
  v4i v[4];
};

__device__ __forceinline__ v4i ldg_b128(const uint8_t* p, bool ok) {
  if (!ok) return v4i{0, 0, 0, 0};
  return *reinterpret_cast<const v4i*>(p);
}

__device__ __forceinline__ uint32_t ldg_u32(const uint8_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
}
__device__ __forceinline__ uint32_t ldg_u8(const uint8_t* p, bool ok) { return ok ? (uint32_t)*p : 0u; }

// 4 consecutive scale bytes of row `rb` starting at block column `kb` (zero past the end).
__device__ __forceinline__ uint32_t load_scale4(const uint8_t* s, int64_t rb, int64_t nrb,
                                                int64_t kb, int64_t nkb, bool vec_ok) {
  if (rb >= nrb) return 0u;
  const uint8_t* p = s + rb * nkb + kb;
  if (vec_ok) return *reinterpret_cast<const uint32_t*>(p);
  uint32_t w = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (kb + q < nkb) w |= (uint32_t)p[q] << (8 * q);
  return w;
}

__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, v16f c, uint32_t sa, uint32_t sb, int s) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  if (s == 0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, (int)sa, 0, (int)sb);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 2, (int)sa, 2, (int)sb);
}

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup -> output tile. Workgroups are dealt round-robin to the 8 XCDs; renumber
// so each XCD gets a contiguous run of tiles, then walk tiles in bands of GROUP_M
// row-tiles so that concurrently running workgroups of one XCD share operand rows in
// its L2.
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int GROUP_M = 4;
  const int band = bid / (GROUP_M * tiles_n);
  const int first_m = band * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int in_band = bid - band * GROUP_M * tiles_n;
  tm = first_m + in_band % gm;
  tn = in_band / gm;
}

template <bool TRANS_B, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void k_gemm_mx4(const GemmArgs g) {
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* smem = (lds_char*)(smem_raw);
  lds_char* sA[2] = {smem, smem + A_TILE_BYTES};
  lds_char* sB[2] = {smem + 2 * A_TILE_BYTES, smem + 2 * A_TILE_BYTES + B_TILE_BYTES};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t Kred = g.Kred;
  const int KT = (int)((Kred + BK - 1) / BK);
  const int64_t a_pitch = Kred >> 1;                        // bytes per A row
  const int64_t nkb_a = Kred >> 5;                          // scale blocks per A row
  const int64_t nrb_a = (g.M + 31) >> 5;
  const bool a_vec = (nkb_a & 3) == 0;

  // ---------------------------------------------------------------- staging helpers
  auto load_a = [&](int kt, Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 2, c16 = c & 3;
      const int64_t gr = m0 + row, gk = (int64_t)kt * BK + c16 * 32;
      f.v[i] = ldg_b128(g.a_codes + gr * a_pitch + (gk >> 1), gr < g.M && gk < Kred);
    }
  };
  auto store_a = [&](lds_char* dst, const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 2, c16 = c & 3;
      lds_write_b128(dst + swz64(row, c16), f.v[i]);
    }
  };
  auto load_b = [&](int kt, Frag& f) {
    if constexpr (!TRANS_B) {
      // B rows are R rows n0.. (reduction over K, K-contiguous)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, row = c >> 2, c16 = c & 3;
        const int64_t gr = n0 + row, gk = (int64_t)kt * BK + c16 * 32;
        f.v[i] = ldg_b128(g.b_codes + gr * g.b_pitch + (gk >> 1), gr < g.N && gk < Kred);
      }
    } else {
      // R rows kt*128 .. +128 (reduction index), 256 output columns n0.. (128 bytes)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, row = c >> 3, c16 = c & 7;
        const int64_t gr = (int64_t)kt * BK + row, gc = n0 + c16 * 32;
        f.v[i] = ldg_b128(g.b_codes + gr * g.b_pitch + (gc >> 1), gr < Kred && gc < g.N);
      }
    }
  };
  auto store_b = [&](lds_char* dst, const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      if constexpr (!TRANS_B)
        lds_write_b128(dst + swz64(c >> 2, c & 3), f.v[i]);
      else
        lds_write_b128(dst + swz128(c >> 3, c & 7), f.v[i]);
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  Frag fa, fb;
  load_a(0, fa);
  load_b(0, fb);
  store_a(sA[0], fa);
  store_b(sB[0], fb);
  __syncthreads();

  const int half = lane >> 5;  // which 32-element half of the 64-step this lane holds
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      load_a(kt + 1, fa);
      load_b(kt + 1, fb);
    }
    // scale bytes of this step: A row-block of each row tile, 4 reduction blocks
    uint32_t sa[TI], sb[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t rb = (m0 + wm * 128 + 32 * i) >> 5;
      sa[i] = load_scale4(g.a_scales, rb, nrb_a, (int64_t)kt * 4, nkb_a, a_vec) >> (8 * half);
    }
    if constexpr (!TRANS_B) {
      const int64_t nkb_b = Kred >> 5, nrb_b = (g.N + 31) >> 5;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t rb = (n0 + wn * 128 + 32 * j) >> 5;
        sb[j] = load_scale4(g.b_scales, rb, nrb_b, (int64_t)kt * 4, nkb_b, (nkb_b & 3) == 0) >> (8 * half);
      }
    } else {
      // reduction blocks kt*4 + {half, 2 + half}; output block column of tile j
      const int64_t nkb_b = g.N >> 5, nrb_b = (Kred + 31) >> 5;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t cb = (n0 + wn * 128 + 32 * j) >> 5;
        const int64_t rb0 = (int64_t)kt * 4 + half, rb1 = rb0 + 2;
        const bool cok = cb < nkb_b;
        sb[j] = ldg_u8(g.b_scales + rb0 * nkb_b + cb, cok && rb0 < nrb_b) |
                (ldg_u8(g.b_scales + rb1 * nkb_b + cb, cok && rb1 < nrb_b) << 16);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i af[TI], bf[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wm * 128 + 32 * i + (lane & 31);
        af[i] = lds_read_b128(sA[cur] + swz64(row, 2 * s + half));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (!TRANS_B) {
          const int row = wn * 128 + 32 * j + (lane & 31);
          bf[j] = lds_read_b128(sB[cur] + swz64(row, 2 * s + half));
        } else {
          // column kc of the tile; rows 64s + 32*half + 16h + (lane&15) of the group
          const int grp = lane >> 4;
          const int kc = wn * 128 + 32 * j + 16 * (grp & 1);
          const int rbase = 64 * s + 32 * (grp >> 1) + (lane & 15);
          const int unit = kc >> 5, sub8 = ((kc >> 4) & 1) << 3;
          v2i h0 = lds_read_tr4(sB[cur] + swz128(rbase, unit) + sub8);
          v2i h1 = lds_read_tr4(sB[cur] + swz128(rbase + 16, unit) + sub8);
          bf[j] = v4i{h0.x, h0.y, h1.x, h1.y};
        }
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_fp4(af[i], bf[j], acc[i][j], sa[i], sb[j], s);
    }
    if (kt + 1 < KT) {
      store_a(sA[cur ^ 1], fa);
      store_b(sB[cur ^ 1], fb);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- up-projection
  // acc += low[rows, 0:rt] * up[cols, 0:rt]^T on bf16 MFMA 32x32x16. `low` is XL (fwd)
  // or GB (bwd), [M x rt] bf16. `up` row q holds rt values: the first up_split from
  // up0 (row stride up0_ld), the rest from up1 (row stride up1_ld).
  const int rt = g.rt;
  for (int t = 0; t < rt; t += 16) {
    const int j0 = t + 8 * half;
    v4i la[TI], ub[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t row = m0 + wm * 128 + 32 * i + (lane & 31);
      la[i] = row < g.M ? *reinterpret_cast<const v4i*>(g.low + row * rt + j0) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t q = n0 + wn * 128 + 32 * j + (lane & 31);
      const bf16_t* p = j0 < g.up_split ? g.up0 + q * g.up0_ld + j0
                                        : g.up1 + q * g.up1_ld + (j0 - g.up_split);
      ub[j] = q < g.N ? *reinterpret_cast<const v4i*>(p) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_bf16(la[i], ub[j], acc[i][j]);
  }

  // ---------------------------------------------------------------- store
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < g.M) {
          if constexpr (OUT_BF16)
            reinterpret_cast<bf16_t*>(g.out)[row * g.ldo + col] = (bf16_t)f32_to_bf16_bits(acc[i][j][r]);
          else
            reinterpret_cast<float*>(g.out)[row * g.ldo + col] = acc[i][j][r];
        }
      }
    }
}

}  // namespace

constexpr size_t GEMM_LDS = 2 * (A_TILE_BYTES + B_TILE_BYTES);

hipError_t launch_gemm_mx4(const GemmArgs& g, bool trans_b, bool out_bf16, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  dim3 grid(tiles), block(256);
  if (!trans_b) {
    if (out_bf16)
      hipLaunchKernelGGL((k_gemm_mx4<false, true>), grid, block, GEMM_LDS, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_mx4<false, false>), grid, block, GEMM_LDS, stream, g);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((k_gemm_mx4<true, true>), grid, block, GEMM_LDS, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_mx4<true, false>), grid, block, GEMM_LDS, stream, g);
  }
  return hipGetLastError();
}

}  // namespace ft
