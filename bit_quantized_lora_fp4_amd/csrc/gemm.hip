// 4-bit backbone GEMMs of the W4A4G4 linear on gfx950 scaled-FP4 MFMA, with the
// low-rank up-projection accumulated into the same accumulators (FourTune §3.3 "LoRA
// Fusion": the 4-bit backbone is fused with the up-projections so the branch outputs
// are summed before one store).
//
//   forward  (TRANS_B = false): Y  = deq Q(X) deq Q(R)^T + XL [B|L2]^T     (§3.1)
//   backward (TRANS_B = true ): dX = deq Q(G) deq Q(R)   + GB [A;L1]       (§3.2)
//
// The activation operand is an MXFP4 tensor [M x Kred] read along its rows. Q(R) is the
// frozen [N x K] weight: the forward reduces over its rows' K; the backward reduces
// over N, i.e. reads Q(R) down its columns. Because the 32x32 block scales are local to
// a block, the backward uses the very same codes and scale bytes: code tiles are staged
// row-major in LDS and read transposed with ds_read_b64_tr_b4 (a 16x16 nibble transpose
// across 16 lanes), and each lane picks the scale byte of the block its 32 reduction
// elements fall in (§3.2: a 4-bit block and its scale are fetched together in either
// orientation, with no dequantize/requantize).
//
// Tiling. A workgroup of 8 waves (two per SIMD) computes a 256 x 256 output tile, each
// wave 128 rows x 64 columns as 2 x 4 tiles of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP4 x
// FP4, one E8M0 scale per lane = per 32 reduction elements); the layout is a template
// parameter (Waves<NWN>), 4 waves of 128 x 128 being the other instance. The reduction advances 256
// elements per step. A step's two code tiles (32 KB each, 128-byte rows: whole cache
// lines) land in one of two LDS stages by direct-to-LDS buffer loads issued during the
// step before, one 1 KB segment per scheduling region so the loads go out between
// MFMAs. (An L2 prefetch of the step after that, one 4-byte load per line, made the
// kernel 4-6% slower at every size: it doubles the cache-line requests a step issues.)
// The block scales
// of the workgroup's rows and columns for the whole reduction are staged into LDS
// once, before the main loop. Each stage is its own LDS object, so the compiler knows
// which loads a fragment read can alias. The up-projection's operands (its first 64
// low-rank columns) arrive the same way: the last step loads them into the stage it
// frees, and their bf16 MFMAs run after the loop.
//
// Operand order. The MFMA's first operand is the Q(R) side (output columns), the second
// the activation side (output rows): a lane's accumulator registers 4g..4g+3 then hold
// four consecutive output columns of one output row, so results leave in 8- or 16-byte
// stores. MFMA layout (32x32x64, FP4): lane l holds row l%32 of an operand and the 32
// reduction elements (l/32)*32 .. +32 of the 64-step, two per byte, even element in
// the low nibble; the scale operand byte chosen by op_sel scales those 32. Accumulator
// register r of lane l is element (8*(r/4) + 4*(l/32) + r%4, l%32) of the 32x32 tile
// (first-operand index, second-operand index). The bf16 MFMA 32x32x16 has the same
// accumulator layout, 8 bf16 per lane at reduction offset (l/32)*8.
#include "common.h"
#include <type_traits>
#include <utility>

#include "gemm.h"

namespace ft {

namespace {

constexpr int BM = 256, BN = 256, BK = 256;    // output tile (rows, cols), reduction step
constexpr int TJ = 4;                          // 32x32 MFMA tiles per wave, activation side
constexpr int SUBSTEPS = BK / 64;              // MFMA reduction substeps per step
constexpr int TILE_BYTES = 256 * BK / 2;       // 32 KB of codes per operand tile per step
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // activation tile + R tile
constexpr int SCALE_BYTES = 8192;              // LDS for the two operands' block scales
constexpr int MAX_NKB = SCALE_BYTES / 2 / 8;   // 8 block rows per operand: Kred <= 16384
#ifndef GEMM_NWN
#define GEMM_NWN 4
#endif

// Wave layout of the 256 x 256 tile: 2 waves along the rows (128 each) and NWN along
// the columns. NWN = 4 (8 waves, two per SIMD, 128 x 64 each): while one wave of a
// SIMD stalls issuing its direct-to-LDS loads the other keeps the matrix pipe busy.
template <int NWN>
struct Waves {
  static constexpr int N = 2 * NWN;                  // waves per workgroup
  static constexpr int NT = 64 * N;                  // threads
  static constexpr int WCOLS = BN / NWN;             // output columns per wave
  static constexpr int TI = WCOLS / 32;              // 32x32 MFMA tiles per wave, R side
  static constexpr int SEGS = TILE_BYTES / 1024 / N; // 1 KB load segments per wave per tile
  static constexpr int SW = 8 * MAX_NKB / 4 / NT;    // scale words staged per thread per operand
};


__device__ __forceinline__ v4i lds_read_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(p);
}
__device__ __forceinline__ void lds_write_b128(lds_char* p, v4i v) {
  *reinterpret_cast<__attribute__((address_space(3))) v4i*>(p) = v;
}

// Stage tiles have 128-byte rows (eight 16-byte units); unit c of row r is stored at
// unit c ^ swz8(r). swz8 is distinct over each parity class of 16 consecutive rows, so
// the 32-row fragment reads and the 16-lane transposed reads meet distinct banks.
__device__ __forceinline__ int swz8(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }
__device__ __forceinline__ int off128(int row, int c16) { return row * 128 + ((c16 ^ swz8(row)) << 4); }

// first operand (R side) and its scale word with op_sel SA; second (activation) with SB
template <int SA, int SB>
__device__ __forceinline__ v16f mfma_fp4(v4i r, v4i x, v16f c, uint32_t sr, uint32_t sx) {
  v8i a8 = {r.x, r.y, r.z, r.w, 0, 0, 0, 0};
  v8i b8 = {x.x, x.y, x.z, x.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SA, (int)sr, SB, (int)sx);
}

// substep s (0..3) of a step: op_sel picks byte s of both scale words
__device__ __forceinline__ v16f mfma_fp4_sub(int s, v4i r, v4i x, v16f c, uint32_t sr, uint32_t sx) {
  switch (s) {
    case 0: return mfma_fp4<0, 0>(r, x, c, sr, sx);
    case 1: return mfma_fp4<1, 1>(r, x, c, sr, sx);
    case 2: return mfma_fp4<2, 2>(r, x, c, sr, sx);
    default: return mfma_fp4<3, 3>(r, x, c, sr, sx);
  }
}

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding, then
// meet the other waves. The wait is the compiler's own s_waitcnt (encoded for gfx9:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at "no wait"), so its counter
// model knows the stage loads have landed and inserts no further wait for them before
// the LDS reads; the barrier's memory clobber keeps LDS accesses from moving across.
// Unlike __syncthreads() it does not drain loads that may stay in flight.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");
}



// One transposed 16x16-nibble LDS read (ds_read_b64_tr_b4) as a builtin, so the
// scheduler may place it among MFMAs.
__device__ __forceinline__ v2i lds_tr4(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}

// Scheduling pattern for NM MFMAs with NR LDS reads of the next substep: the reads go
// in among the first NM/2 MFMAs, as evenly as the counts allow.
template <int N>
__device__ __forceinline__ void sched_ds_reads() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
}
template <int NR, int NM, int... K>
__device__ __forceinline__ void sched_mix_impl(std::integer_sequence<int, K...>) {
  constexpr int H = NM / 2;
  ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
    sched_ds_reads<(K < H ? NR * (K + 1) / H - NR * K / H : 0)>()), ...);
}
template <int NR, int NM>
__device__ __forceinline__ void sched_mix() {
  sched_mix_impl<NR, NM>(std::make_integer_sequence<int, NM>{});
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

// One 32x32 accumulator tile = one 32x32 block of the output. Quantize the fp32 values
// v (accumulator layout: lane l holds row l%32, register 4g+c column 8g + 4(l/32) + c)
// to MXFP4 and store codes and the scale byte. Lanes l and l+32 first trade column
// groups with v_permlane32_swap so that lane l holds columns 0..15 of its row and lane
// l+32 columns 16..31: each lane then writes 8 contiguous code bytes.
__device__ __forceinline__ void quant_tile_store(const float (&v)[16], int lane, int64_t row, bool row_ok,
                                                 bool blk_ok, int64_t blk_row, int64_t col0, bufres rcodes,
                                                 bufres rscales, int64_t cpitch, int64_t nkb) {
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = umax(m, __builtin_bit_cast(uint32_t, v[r]) & 0x7FFFFFFFu);
  const uint32_t sb = scale_byte_from_amax(wave_max_u32(m));
  const float scale = e8m0_to_f32_scale(sb);
  float w[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // (g0, g2) and (g1, g3): lanes 32..63 of the first take lanes 0..31 of the second
    const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[c]),
                                                    __builtin_bit_cast(uint32_t, v[8 + c]), false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[4 + c]),
                                                    __builtin_bit_cast(uint32_t, v[12 + c]), false, false);
    w[c] = __builtin_bit_cast(float, (uint32_t)p[0]);
    w[4 + c] = __builtin_bit_cast(float, (uint32_t)p[1]);
    w[8 + c] = __builtin_bit_cast(float, (uint32_t)q[0]);
    w[12 + c] = __builtin_bit_cast(float, (uint32_t)q[1]);
  }
  v2i cw = {(int)cvt8_f32(w, scale), (int)cvt8_f32(w + 8, scale)};
  if (sb == 0xFFu) cw = v2i{0, 0};
  const int half = lane >> 5;
  buf_store8(rcodes, sel_off(row_ok && blk_ok, (uint32_t)(row * cpitch + ((col0 + 16 * half) >> 1))), cw);
  buf_store1(rscales, sel_off(blk_ok && lane == 0, (uint32_t)(blk_row * nkb + (col0 >> 5))), sb);
}

template <bool TRANS_B, bool OUT_BF16, int EPI, int NWN>
__global__ __launch_bounds__(Waves<NWN>::NT, 1) void k_gemm_mx4(const GemmArgs g) {
  using W = Waves<NWN>;
  constexpr int TI = W::TI, SEGS = W::SEGS, SW = W::SW, NT = W::NT;
  constexpr int WCOLS = W::WCOLS;
  // Separate LDS objects per stage: the compiler then knows a transposed LDS read of one
  // stage cannot alias the direct-to-LDS loads still filling the other, and does not
  // drain those loads before the read.
  __shared__ __align__(16) char st0_raw[STAGE_BYTES];
  __shared__ __align__(16) char st1_raw[STAGE_BYTES];
  __shared__ __align__(16) char scale_raw[SCALE_BYTES];
  lds_char* const st0 = (lds_char*)st0_raw;
  lds_char* const st1 = (lds_char*)st1_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;  // wave's half of the tile rows, its column slice
  const int half = lane >> 5;               // which 32-element half of a 64-step this lane holds
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  const int ntile = tiles_m * tiles_n;
  if ((int)blockIdx.x >= ntile) {
    // a workgroup past the output tiles: its share of the LoRA-gradient row-range sum
    const int64_t nthr = (int64_t)(gridDim.x - ntile) * NT;
    for (int64_t i = (int64_t)(blockIdx.x - ntile) * NT + tid; i < g.tail.items; i += nthr) lora_reduce_item(g.tail, i);
    return;
  }
  int tm, tn;
  tile_of(blockIdx.x, ntile, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t Kred = g.Kred;
  const int KT = (int)((Kred + BK - 1) / BK);

  const int64_t a_pitch = Kred >> 1;                    // bytes per activation row
  const int64_t nkb = Kred >> 5;                        // scale blocks per reduction row
  const int64_t nrb_a = (g.M + 31) >> 5;
  const int64_t r_rows = TRANS_B ? Kred : g.N;          // rows of Q(R)
  const int64_t nkb_r = TRANS_B ? (g.N >> 5) : nkb;     // scale bytes per R block row
  const bool vec_scales = (nkb & 7) == 0;

  const bufres ra = make_buf(g.a_codes, (uint64_t)g.M * a_pitch);
  const bufres rsa = make_buf(g.a_scales, (uint64_t)nrb_a * nkb);
  const bufres rr = make_buf(g.b_codes, (uint64_t)r_rows * g.b_pitch);
  const bufres rsr = make_buf(g.b_scales, (uint64_t)((r_rows + 31) >> 5) * nkb_r);

  // ---- per-lane DMA sources: segment q (1 KB) of a tile; lane l fills the 16-byte LDS
  // slot 16*l of the segment. Every tile has 128-byte rows (whole cache lines):
  //   activation / forward-R tile: 256 rows x 256 reduction elements
  //   backward-R tile: 256 reduction rows x 256 output columns
  // rows 8q + l/8, slot unit l%8, holding global unit (l%8) ^ swz8(row).
  uint32_t a_base[SEGS], r_base[SEGS];
  bool a_ok[SEGS], r_ok[SEGS];
  int a_k[SEGS], r_k[SEGS];  // reduction offset within the step (elements)
#pragma unroll
  for (int i = 0; i < SEGS; ++i) {
    const int q = wave * SEGS + i;
    {
      const int row = 8 * q + (lane >> 3), c16 = (lane & 7) ^ swz8(row);
      a_k[i] = c16 * 32;
      a_ok[i] = m0 + row < g.M;
      a_base[i] = (uint32_t)((m0 + row) * a_pitch + c16 * 16);
    }
    if constexpr (!TRANS_B) {
      const int row = 8 * q + (lane >> 3), c16 = (lane & 7) ^ swz8(row);
      r_k[i] = c16 * 32;
      r_ok[i] = n0 + row < g.N;
      r_base[i] = (uint32_t)((n0 + row) * g.b_pitch + c16 * 16);
    } else {
      const int row = 8 * q + (lane >> 3), c16 = (lane & 7) ^ swz8(row);
      r_k[i] = row;
      r_ok[i] = n0 + c16 * 32 < g.N;
      r_base[i] = (uint32_t)(row * g.b_pitch + (n0 >> 1) + c16 * 16);
    }
  }
  // segment i of the activation tile (part 0) or of the R tile (part 1)
  // The stage loads' sources are loop-carried: before the last step they are switched
  // to the up-projection's operands (switch_to_low below), which that step then loads
  // into the stage it frees. Past the reduction's end the offsets go out of range, so
  // no step needs a "live" test of its own.
  bufres src_a = ra, src_r = rr;
  int kred_eff = (int)Kred;
  auto issue_part = [&](lds_char* st, int kt, int i, int part) __attribute__((always_inline)) {
    const int q = wave * SEGS + i;
    if (part == 0) {
      const bool ka = a_ok[i] && kt * BK + a_k[i] < kred_eff;
      buf_load16_lds(src_a, st + q * 1024, sel_off(ka, a_base[i] + (uint32_t)kt * (BK / 2)));
    } else {
      const bool kr = r_ok[i] && kt * BK + r_k[i] < kred_eff;
      uint32_t ro;
      if constexpr (!TRANS_B) ro = r_base[i] + (uint32_t)kt * (BK / 2);
      else ro = r_base[i] + (uint32_t)((int64_t)kt * BK * g.b_pitch);
      buf_load16_lds(src_r, st + TILE_BYTES + q * 1024, sel_off(kr, ro));
    }
  };
  auto issue_stage = [&](lds_char* st, int kt) {
#pragma unroll
    for (int i = 0; i < SEGS; ++i) {
      issue_part(st, kt, i, 0);
      issue_part(st, kt, i, 1);
    }
  };

  // ---- block scales for the whole reduction, staged once, step-major: for step kt,
  // lane half h and block row b (0..7) of the tile's operand, the word at
  //   64*kt + 32*h + 4*b
  // holds, in byte s, the scale of reduction block 8*kt + 2*s + h: exactly what lane
  // half h needs in substep s (op_sel picks byte s). A wave reads its four block rows
  // of a step with one 16-byte read per operand. The R side of the backward is the
  // transposed scale matrix (block row b = output block). The loads are issued before
  // the first stages' and written to LDS after them, so their latency overlaps.
  const int sp = (int)((nkb + 7) & ~7);  // a step reads 8 scale bytes (two words)
  lds_char* sSA = (lds_char*)scale_raw;
  lds_char* sSR = sSA + SCALE_BYTES / 2;
  const int wpr = sp / 4;  // words per staged row
  constexpr int SKB = MAX_NKB / NT > 0 ? MAX_NKB / NT : 1;  // backward scale rows per thread
  uint32_t sa_w[SW], sr_w[SW], st_lo[SKB], st_hi[SKB];
  auto word = [&](bufres res, int64_t row, bool row_ok, int64_t pitch, int kw) -> uint32_t {
    // bytes 4kw .. 4kw+3 of a scale row, zero past the row end
    const int64_t o = row * pitch + 4 * kw;
    if ((pitch & 3) == 0) return buf_load4(res, (row_ok && 4 * kw < pitch) ? (uint32_t)o : BUF_OOB);
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w |= buf_load1(res, (row_ok && 4 * kw + q < pitch) ? (uint32_t)(o + q) : BUF_OOB) << (8 * q);
    return w;
  };
#pragma unroll
  for (int u = 0; u < SW; ++u) {
    const int e = tid + NT * u, blk = e / max(wpr, 1), kw = e % max(wpr, 1);
    const bool live = e < 8 * wpr;
    const int64_t arb = (m0 >> 5) + blk;
    sa_w[u] = word(rsa, arb, live && arb < nrb_a, nkb, kw);
    if constexpr (!TRANS_B) {
      const int64_t rrb = (n0 >> 5) + blk;
      sr_w[u] = word(rsr, rrb, live && rrb < ((g.N + 31) >> 5), nkb, kw);
    }
  }
  if constexpr (TRANS_B) {
    // scale row kb (reduction block) holds output blocks cb0 .. cb0+7 in 8 bytes
#pragma unroll
    for (int u = 0; u < SKB; ++u) {
      const int kb = tid + NT * u;
      const bool live = kb < nkb;
      const int64_t o = (int64_t)kb * nkb_r + (n0 >> 5);
      if ((nkb_r & 3) == 0) {
        st_lo[u] = buf_load4(rsr, live ? (uint32_t)o : BUF_OOB);
        st_hi[u] = buf_load4(rsr, live ? (uint32_t)(o + 4) : BUF_OOB);
      } else {
        st_lo[u] = st_hi[u] = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t b = buf_load1(rsr, (live && (n0 >> 5) + q < nkb_r) ? (uint32_t)(o + q) : BUF_OOB);
          if (q < 4) st_lo[u] |= b << (8 * q);
          else st_hi[u] |= b << (8 * (q - 4));
        }
      }
    }
  }
  // reduction blocks 4kw .. 4kw+3 of block row b: bytes 0, 2 go to half 0 and bytes
  // 1, 3 to half 1, each pair at substeps 2(kw%2), 2(kw%2)+1 of step kw/2
  // The staging stores are written from inline asm: they run while stage 0 is in
  // flight, and the compiler, seeing plain LDS stores there, would wait for every
  // load in flight first. Their
  // completion is awaited by the lgkmcnt wait before the barrier that follows.
  auto put_word = [&](lds_char* dst, int b, int kw, uint32_t w) {
    const uint32_t o = (uint32_t)(uintptr_t)(dst + 64 * (kw >> 1) + 4 * b + 2 * (kw & 1));
    const uint32_t lo = (w & 0xFFu) | ((w >> 8) & 0xFF00u), hi = ((w >> 8) & 0xFFu) | ((w >> 16) & 0xFF00u);
    asm volatile("ds_write_b16 %0, %1\n\tds_write_b16 %0, %2 offset:32" ::"v"(o), "v"(lo), "v"(hi) : "memory");
  };
  auto write_scales = [&]() {
#pragma unroll
    for (int u = 0; u < SW; ++u) {
      const int e = tid + NT * u, blk = e / max(wpr, 1), kw = e % max(wpr, 1);
      if (e < 8 * wpr) {
        put_word(sSA, blk, kw, sa_w[u]);
        if constexpr (!TRANS_B) put_word(sSR, blk, kw, sr_w[u]);
      }
    }
    if constexpr (TRANS_B) {
#pragma unroll
      for (int u = 0; u < SKB; ++u) {
        const int kb = tid + NT * u;
        if (kb < sp) {  // rows kb in [nkb, sp) are the zero padding
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t o = (uint32_t)(uintptr_t)(sSR + 64 * (kb >> 3) + 32 * (kb & 1) + 4 * q + ((kb >> 1) & 3));
            const uint32_t v = ((q < 4 ? st_lo[u] : st_hi[u]) >> (8 * (q & 3))) & 0xFFu;
            asm volatile("ds_write_b8 %0, %1" ::"v"(o), "v"(v) : "memory");
          }
        }
      }
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  // ---- one reduction step of MFMAs, four 64-element substeps. Fragments are double-
  // buffered in registers: substep s+1's LDS reads are issued between substep s's MFMAs
  // (sched_group_barrier pins the interleave), so LDS latency hides behind the matrix
  // pipe instead of stalling it once per fragment. A 32-bit scale read gives two
  // substeps' blocks; shifted by this lane's half, substep s's byte sits at position
  // 2*(s%2) (op_sel).
  struct Frag {
    v4i x[TJ], r[TI];
  };
  // backward: this lane's byte offset of fragment 0 within an R tile, for the
  // transposed reads (row 32*half + (lane&15), unit TI*wn, byte 8*(lane/16 % 2) of the
  // unit). Kept opaque so each read's address stays one step from its stage: the
  // compiler then knows which LDS object it reads and that in-flight loads into the
  // other stage cannot alias it.
  uint32_t frag_tr = 0;
  if constexpr (TRANS_B) {
    const int rb = 32 * half + (lane & 15);
    frag_tr = (uint32_t)(rb * 128 + (((TI * wn) ^ swz8(rb)) << 4) + ((lane >> 4) & 1) * 8);
    asm("" : "+v"(frag_tr));
  }
  auto load_x = [&](const lds_char* st, int s, int j) __attribute__((always_inline)) -> v4i {
    const int row = wm * 128 + 32 * j + (lane & 31);
    return lds_read_b128(st + off128(row, 2 * s + half));
  };
  auto load_r = [&](const lds_char* st, int s, int i) __attribute__((always_inline)) -> v4i {
    if constexpr (!TRANS_B) {
      const int row = wn * WCOLS + 32 * i + (lane & 31);
      return lds_read_b128(st + TILE_BYTES + off128(row, 2 * s + half));
    } else {
      const uint32_t o = frag_tr ^ (uint32_t)(i << 4);
      const v2i lo = lds_tr4(st + (TILE_BYTES + 8192 * s) + o);
      const v2i hi = lds_tr4(st + (TILE_BYTES + 8192 * s + 2048) + o);
      return v4i{lo.x, lo.y, hi.x, hi.y};
    }
  };
  auto load_frag = [&](const lds_char* st, int s, Frag& f) __attribute__((always_inline)) {
    const lds_char* sX = st;
    const lds_char* sR = st + TILE_BYTES;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wm * 128 + 32 * j + (lane & 31);
      f.x[j] = lds_read_b128(sX + off128(row, 2 * s + half));
    }
    if constexpr (!TRANS_B) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wn * WCOLS + 32 * i + (lane & 31);
        f.r[i] = lds_read_b128(sR + off128(row, 2 * s + half));
      }
    } else {
      // output column c = wn*WCOLS + 32i + (lane&31); reduction rows
      // 64s + 32*half + 16h + (lane&15): two 16x16 nibble transposes per fragment.
      // off128(64s + 16h + rb, unit) = off128(rb, unit) + 8192s + 2048h (swz8 ignores
      // row bits 3 and up), and fragment i's unit is TI*wn + i, so its offset is the
      // lane's base with i XORed into the unit field.
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint32_t o = frag_tr ^ (uint32_t)(i << 4);
        const v2i lo = lds_tr4(st + (TILE_BYTES + 8192 * s) + o);
        const v2i hi = lds_tr4(st + (TILE_BYTES + 8192 * s + 2048) + o);
        f.r[i] = v4i{lo.x, lo.y, hi.x, hi.y};
      }
    }
  };
  auto load_scales = [&](int kt, uint32_t (&xs)[TJ], uint32_t (&rs)[TI]) {
    const v4i a = lds_read_b128(sSA + 64 * kt + 32 * half + 16 * wm);
    xs[0] = a.x, xs[1] = a.y, xs[2] = a.z, xs[3] = a.w;
    if constexpr (TI == 4) {
      const v4i r = lds_read_b128(sSR + 64 * kt + 32 * half + 16 * wn);
      rs[0] = r.x, rs[1] = r.y, rs[2] = r.z, rs[3] = r.w;
    } else {
      const v2i r = *reinterpret_cast<const __attribute__((address_space(3))) v2i*>(sSR + 64 * kt + 32 * half + 4 * TI * wn);
      rs[0] = r.x, rs[1] = r.y;
    }
  };
  // ---- operands of the up-projection's first 64 low-rank columns. They are loaded by
  // the last reduction step into the stage it frees, in place of a next step's codes,
  // so their latency hides behind that step's MFMAs (loaded ahead of stage 0 instead,
  // they delayed the first step by their own round trip). `low` = XL (forward) or GB
  // (backward), [M x rt] bf16; the up side is [B | L2] rows (forward, row = output
  // column; the first up_split values from up0, row stride up0_ld, the rest from up1)
  // or [A; L1] rows (backward, row j = reduction index: up0 row j for j < up_split,
  // else up1 row j - up_split). Stage layouts:
  //   low side and forward up side: unit-major, the 16-byte unit c (low-rank columns
  //   8c .. 8c+7) of tile row r at 4096c + 16r, one load instruction per 64 rows of a
  //   unit; rank and stab_rank are multiples of 16, so a unit never straddles the two
  //   sources and every instruction reads one tensor;
  //   backward up side: rows j = 0..63 of the tile's 256 columns, row-major, 512 bytes
  //   per row (read transposed with ds_read_b64_tr_b16).
  const int rt = g.rt;
  const int rt1 = rt < 64 ? rt : 64;
  const bufres rl = make_buf(g.low, (uint64_t)g.M * rt * 2);
  const bufres ru0 = TRANS_B ? make_buf(g.up0, (uint64_t)g.up_split * g.up0_ld * 2)
                             : make_buf(g.up0, (uint64_t)g.N * g.up0_ld * 2);
  const bufres ru1 = TRANS_B ? make_buf(g.up1, (uint64_t)(rt - g.up_split) * g.up1_ld * 2)
                             : make_buf(g.up1, (uint64_t)g.N * g.up1_ld * 2);
  constexpr int DP1 = BN * 2;  // row pitch of the backward up side (bytes)
  // Per-lane parts of those loads' offsets; the rest of each offset is wave-uniform
  // (segment q = SEGS wave + i: unit c = q/4, rows 64 (q%4) .. +64; SEGS is a multiple
  // of 4, so q%4 = i%4).
  const int lim_m = (int)min<int64_t>(g.M - m0, BM), lim_n = (int)min<int64_t>(g.N - n0, BN);
  const uint32_t low_base = (uint32_t)(2 * (m0 + lane) * rt);
  uint32_t up_base0, up_base1;
  if constexpr (!TRANS_B) {
    up_base0 = (uint32_t)(2 * (n0 + lane) * g.up0_ld);
    up_base1 = (uint32_t)(2 * (n0 + lane) * g.up1_ld);
  } else {
    up_base0 = (uint32_t)(2 * ((lane >> 5) * g.up0_ld + n0 + 8 * (lane & 31)));
    up_base1 = (uint32_t)(2 * ((lane >> 5) * g.up1_ld + n0 + 8 * (lane & 31)));
  }
  // Point the stage loads at the up-projection's operands: issue_part(st, KT, i, part)
  // then loads segment q = SEGS wave + i of the low side (part 0) or the up side (part 1).
  // Every segment of a wave draws from one source tensor: its up-side units (forward)
  // or row pairs (backward) cover rank columns 2 SEGS wave .. +2 SEGS, and up_split is
  // a multiple of 16 >= 2 SEGS.
  auto switch_to_low = [&]() {
    const bool first = 2 * SEGS * wave < g.up_split;
    src_a = rl;
    src_r = first ? ru0 : ru1;
    kred_eff = 1 << 30;  // the reduction-range test passes; a_ok / r_ok decide
    const uint32_t back_a = (uint32_t)KT * (BK / 2);
    const uint32_t back_r = TRANS_B ? (uint32_t)((int64_t)KT * BK * g.b_pitch) : back_a;
#pragma unroll
    for (int i = 0; i < SEGS; ++i) {
      const int q = wave * SEGS + i;
      a_ok[i] = lane + 64 * (i & 3) < lim_m && 8 * (q >> 2) < rt1;
      a_base[i] = low_base + (uint32_t)(128 * (i & 3) * rt + 16 * (q >> 2)) - back_a;
      if constexpr (!TRANS_B) {
        const int t = 8 * (q >> 2);
        r_ok[i] = lane + 64 * (i & 3) < lim_n && t < rt1;
        r_base[i] = (first ? up_base0 + (uint32_t)(128 * (i & 3) * g.up0_ld + 2 * t)
                           : up_base1 + (uint32_t)(128 * (i & 3) * g.up1_ld + 2 * (t - g.up_split))) - back_r;
      } else {
        // lane halves take rows j = 2q and 2q+1; rt1 is even, so both rows are live
        // exactly when 2q < rt1
        r_ok[i] = 8 * (lane & 31) < lim_n && 2 * q < rt1;
        r_base[i] = (first ? up_base0 + (uint32_t)(4 * q * g.up0_ld)
                           : up_base1 + (uint32_t)(2 * (2 * q - g.up_split) * g.up1_ld)) - back_r;
      }
    }
  };

  // One step in 16 scheduling regions of 4 MFMAs (one R fragment against the four
  // activation fragments). Region (s, q) also issues the LDS reads of fragments q of
  // substep s+1 and one 1 KB segment of step kt+1's stage (activation and R segments
  // alternating): the direct-to-LDS loads go out one per region between MFMAs instead
  // of all at once ahead of them (a wave stalls at issue while the load queue is full,
  // and could not start its MFMAs until its last load was accepted). Spread over the
  // whole step they cost less than they lose in lead time (measured: 16 loads up
  // front 2.08 us per step, over two substeps 1.74, over four 1.68 at c2).
  auto compute = [&](const lds_char* st, int kt, lds_char* nxt) __attribute__((always_inline)) {
    Frag f[2];
    uint32_t xs[TJ], rs[TI];
    load_scales(kt, xs, rs);
    load_frag(st, 0, f[0]);
#pragma unroll
    for (int s = 0; s < SUBSTEPS; ++s) {
      const Frag& c = f[s & 1];
      Frag& nf = f[(s + 1) & 1];
#pragma unroll
      for (int q = 0; q < TI; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        // the region's loads first (in program order: the empty asm statements that
        // pin the MFMAs also fence the scheduler), then its four MFMAs
        issue_part(nxt, kt + 1, (TI * s + q) >> 1, q & 1);
        if (s + 1 < SUBSTEPS) {
#pragma unroll
          for (int jj = 0; jj < TJ / TI; ++jj) nf.x[q * (TJ / TI) + jj] = load_x(st, s + 1, q * (TJ / TI) + jj);
          nf.r[q] = load_r(st, s + 1, q);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[q][j] = mfma_fp4_sub(s, c.r[q], c.x[j], acc[q][j], rs[q], xs[j]);
          asm volatile("" : "+a"(acc[q][j]));  // keeps the MFMA in this region (no sinking)
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };


  // ---------------------------------------------------------------- up-projection helpers
  // acc += up * low^T on bf16 MFMA 32x32x16 (first operand the output-column side).
  // Forward slices past the first 64 low-rank columns read their operands straight
  // from memory.
  auto up_loads_fwd = [&](int t0, v4i (&la)[4][TJ], v4i (&ub)[4][TI]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 16 * u, j0 = t + 8 * half;
      const bool live = t < rt;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t row = m0 + wm * 128 + 32 * j + (lane & 31);
        la[u][j] = buf_load16(rl, sel_off(live, (uint32_t)((row * rt + j0) * 2)));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t q = n0 + wn * WCOLS + 32 * i + (lane & 31);
        ub[u][i] = (live && t < g.up_split) ? buf_load16(ru0, (uint32_t)((q * g.up0_ld + j0) * 2))
                                            : buf_load16(ru1, sel_off(live, (uint32_t)((q * g.up1_ld + j0 - g.up_split) * 2)));
      }
    }
  };
  auto up_mfma_fwd = [&](int t0, const v4i (&la)[4][TJ], const v4i (&ub)[4][TI]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (t0 + 16 * u >= rt) break;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_bf16(ub[u][i], la[u][j], acc[i][j]);
    }
  };
  // The first 64 low-rank columns from the stage `st` the last step filled (layouts at
  // issue_low). Forward up operand: 8 consecutive columns of one row, a 16-byte read.
  // Backward: 8 consecutive rows j of one output column, two transposed 16-bit reads
  // (lds_tr16_pair's lane pattern, addresses one step from the stage object so the
  // compiler sees which LDS object they read).
  auto up_lds = [&](const lds_char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (16 * u >= rt1) break;
      v4i la[TJ], ub[TI];
#pragma unroll
      for (int j = 0; j < TJ; ++j) la[j] = lds_read_b128(st + (2 * u + half) * 4096 + (wm * 128 + 32 * j + (lane & 31)) * 16);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if constexpr (!TRANS_B) {
          ub[i] = lds_read_b128(st + TILE_BYTES + (2 * u + half) * 4096 + (wn * WCOLS + 32 * i + (lane & 31)) * 16);
        } else {
          const int gq = lane >> 4, sq = lane & 15;
          const int col = wn * WCOLS + 32 * i + 16 * (gq & 1) + 4 * (sq & 3);
          const int m = 16 * u + 8 * (gq >> 1) + (sq >> 2);
          const int o = m * DP1 + col * 2;
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(st + (TILE_BYTES + o)));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(st + (TILE_BYTES + o + 4 * DP1)));
          ub[i] = v4i{(int)(((uint32_t)(uint16_t)lo.x) | ((uint32_t)(uint16_t)lo.y << 16)),
                      (int)(((uint32_t)(uint16_t)lo.z) | ((uint32_t)(uint16_t)lo.w << 16)),
                      (int)(((uint32_t)(uint16_t)hi.x) | ((uint32_t)(uint16_t)hi.y << 16)),
                      (int)(((uint32_t)(uint16_t)hi.z) | ((uint32_t)(uint16_t)hi.w << 16))};
        }
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_bf16(ub[i], la[j], acc[i][j]);
    }
  };
  constexpr int DP = BN * 2 + 32;  // slab row pitch (bytes) of the backward's later slabs
  auto slab_unit = [&](int jc, int c) __attribute__((always_inline)) -> v4i {
    const int row = c >> 5, c16 = c & 31;
    const int j = jc + row;
    const int64_t col = n0 + 8 * c16;
    const bool ok = col < g.N && j < rt;
    // both sources are read (the other one at an out-of-range offset, which returns
    // zeros), so the row's source is a select, not a branch around each load
    const bool first = j < g.up_split;
    return buf_load16(ru0, sel_off(ok && first, (uint32_t)(((int64_t)j * g.up0_ld + col) * 2))) |
           buf_load16(ru1, sel_off(ok && !first, (uint32_t)(((int64_t)(j - g.up_split) * g.up1_ld + col) * 2)));
  };
  // ---------------------------------------------------------------- main loop
  // Two stages: step kt+1's 64 KB land while step kt is multiplied.
  issue_stage(st0, 0);
  asm volatile("" ::: "memory");
  write_scales();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the staging stores are done
  vm_barrier<0>();  // step 0 landed; scales in LDS
  // One step: step kt+1's loads go into the stage step kt-1 used (every wave left it at
  // the last barrier), then step kt's MFMAs run while they land. Unrolled by two so each
  // step names its stage statically. The last step loads the up-projection's operands.
  auto step = [&](lds_char* cur, lds_char* nxt, int kt) __attribute__((always_inline)) {
    compute(cur, kt, nxt);  // also issues step kt+1's stage loads into nxt
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    vm_barrier<0>();
  };
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + 1 == KT) switch_to_low();
    step(st0, st1, kt);
    if (kt + 1 < KT) {
      if (kt + 2 == KT) switch_to_low();
      step(st1, st0, kt + 1);
    }
  }
  if (rt > 0) up_lds((KT & 1) ? st1 : st0);

  // ---------------------------------------------------------------- up-projection, part 2
  if constexpr (!TRANS_B) {
    // forward, rt > 64: the remaining 64-wide slices (the first came with the last step)
    for (int t0 = 64; t0 < rt; t0 += 64) {
      v4i la[4][TJ], ub[4][TI];
      up_loads_fwd(t0, la, ub);
      up_mfma_fwd(t0, la, ub);
    }
  } else {
    // backward, rt > 64: the remaining 32-row slabs of up = [A; L1] [rt x N] (row j =
    // up0 row j for j < up_split, else up1 row j - up_split; the first 64 came with the
    // last step). The MFMA wants 8 consecutive j per output column, so each slab of
    // the tile's 256 columns is staged in LDS (free after the main loop, once every
    // wave has read the first 64 rows' stage) and read transposed with
    // ds_read_b64_tr_b16.
    if (rt > 64) __syncthreads();
    for (int jc = 64; jc < rt; jc += 32) {
      v4i la[2][TJ];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int64_t row = m0 + wm * 128 + 32 * j + (lane & 31);
          la[u][j] = buf_load16(rl, (uint32_t)((row * rt + jc + 16 * u + 8 * half) * 2));
        }
#pragma unroll
      for (int i = 0; i < 1024 / NT; ++i) {
        const int c = tid + NT * i;
        lds_write_b128(st0 + (c >> 5) * DP + (c & 31) * 16, slab_unit(jc, c));
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        v4i ub[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) ub[i] = lds_tr16_pair(st0, DP, 16 * u, wn * WCOLS + 32 * i, lane);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_bf16(ub[i], la[u][j], acc[i][j]);
      }
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- MLP epilogues
  // backward (FC2's dX GEMM): dP = dH * GELU'(P^) in place, Q(dP) from the fp32 values;
  // the store below then writes bf16(dP). (dH exists only here, in fp32: moving this
  // step out of the GEMM would mean storing dH.)
  if constexpr (EPI == GEMM_EPI_DGELU_Q) {
    const bufres rqc = make_buf(g.q_codes, (uint64_t)g.M * (g.N >> 1));
    const bufres rqs = make_buf(g.q_scales, (uint64_t)((g.M + 31) >> 5) * (g.N >> 5));
    const bufres rpre = make_buf(g.pre, (uint64_t)g.M * g.N * 2);
    // P^ is requested two block rows ahead (32 loads in flight), so the tiles below
    // wait for their loads in turn instead of one round trip each
    v2i pw[2][TI][4];
    auto load_pre = [&](int j, v2i (&dst)[TI][4]) __attribute__((always_inline)) {
      const int64_t row = m0 + wm * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int64_t col = n0 + wn * WCOLS + 32 * i + 8 * gq + 4 * half;
          dst[i][gq] = buf_load8(rpre, sel_off(row < g.M && col < g.N, (uint32_t)((row * g.N + col) * 2)));
        }
    };
    load_pre(0, pw[0]);
    load_pre(1, pw[1]);
    const bool dbg = g.dbg != nullptr;  // uniform
    const bufres rdbg = make_buf(g.dbg, dbg ? (uint64_t)g.M * g.N * 4 : 0);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t brow = m0 + wm * 128 + 32 * j;  // first row of this block row
      const int64_t row = brow + (lane & 31);
      const bool row_ok = row < g.M;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t col0 = n0 + wn * WCOLS + 32 * i;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t pwd = (uint32_t)((r & 2) ? pw[j & 1][i][r >> 2].y : pw[j & 1][i][r >> 2].x);
          const float p = (r & 1) ? bf16_hi(pwd) : bf16_lo(pwd);
          acc[i][j][r] = acc[i][j][r] * gelu_grad_f(p);  // dP = dH * GELU'(P^)
          v[r] = acc[i][j][r];
        }
        if (dbg) {  // optional export of the fp32 dP that Q(dP) quantizes
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int64_t col = col0 + 8 * gq + 4 * half;
            buf_store16(rdbg, sel_off(row_ok && col < g.N, (uint32_t)((row * g.N + col) * 4)),
                        __builtin_bit_cast(v4i, v4f{v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]}));
          }
        }
        quant_tile_store(v, lane, row, row_ok, brow < g.M && col0 < g.N, brow >> 5, col0, rqc, rqs, g.N >> 1,
                         g.N >> 5);
        __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounded register use
      }
      if (j + 2 < TJ) load_pre(j + 2, pw[j & 1]);
    }
  }

  // ---------------------------------------------------------------- store
  // Each wave stages its 128 x WCOLS result in LDS (the stages are free now: 32 KB per
  // wave with 4 waves, 16 KB with 8), then consecutive lanes write whole rows of it,
  // 16 bytes each. acc[i][j]: lane holds output row 32j + l%32 of the wave tile and, in
  // registers 4g..4g+3, columns 32i + 8g + 4*half .. +4. Staged rows are 2 WCOLS bytes
  // (bf16) or 4 WCOLS (fp32, 64 rows per pass) with 16-byte units XOR-swizzled by the
  // row, so column reads across rows and row reads across units both spread over the
  // banks.
  __syncthreads();
  constexpr int WB = 2 * STAGE_BYTES / W::N;
  lds_char* wbuf = (wave < W::N / 2 ? st0 : st1) + (wave % (W::N / 2)) * WB;
  constexpr int RB = 2 * WCOLS, UB = RB / 16;       // bf16 staged row
  constexpr int RBF = 4 * WCOLS, UBF = RBF / 16;    // fp32 staged row
  auto wofs = [](int r, int byte) { return r * RB + ((((byte >> 4) ^ r) & (UB - 1)) << 4) + (byte & 15); };
  auto wofs_f = [](int r, int byte) { return r * RBF + ((((byte >> 4) ^ r) & (UBF - 1)) << 4) + (byte & 15); };
  const int64_t orow0 = m0 + wm * 128, ocol0 = n0 + wn * WCOLS;
  if constexpr (OUT_BF16) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = 32 * j + (lane & 31);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const v16f& a = acc[i][j];
          const v2i v = {(int)pack_bf16x2(a[4 * gq], a[4 * gq + 1]),
                         (int)pack_bf16x2(a[4 * gq + 2], a[4 * gq + 3])};
          *(__attribute__((address_space(3))) v2i*)(wbuf + wofs(r, (32 * i + 8 * gq + 4 * half) * 2)) = v;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
    constexpr int RPI = 64 / UB;  // rows per instruction
#pragma unroll 4
    for (int k = 0; k < 128 / RPI; ++k) {
      const int r = RPI * k + lane / UB, c = (lane % UB) * 8;
      const v4i v = lds_read_b128(wbuf + wofs(r, c * 2));
      const int64_t row = orow0 + r, col = ocol0 + c;
      if (row < g.M && col < g.N)  // streaming store: the output is not re-read here
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(reinterpret_cast<bf16_t*>(g.out) + row * g.ldo + col));
    }
  } else {
    // fp32: two passes of 64 rows
    constexpr int RPI = 64 / UBF;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * p + jj;
        const int r = 32 * jj + (lane & 31);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const v16f& a = acc[i][j];
            *(__attribute__((address_space(3))) v4f*)(wbuf + wofs_f(r, (32 * i + 8 * gq + 4 * half) * 4)) =
                v4f{a[4 * gq], a[4 * gq + 1], a[4 * gq + 2], a[4 * gq + 3]};
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
      for (int k = 0; k < 64 / RPI; ++k) {
        const int r = RPI * k + lane / UBF, c = (lane % UBF) * 4;
        const v4i v = lds_read_b128(wbuf + wofs_f(r, c * 4));
        const int64_t row = orow0 + 64 * p + r, col = ocol0 + c;
        if (row < g.M && col < g.N)
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(reinterpret_cast<float*>(g.out) + row * g.ldo + col));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

}  // namespace

static_assert(GEMM_MAX_KRED == MAX_NKB * 32, "scale staging bound");

// Workgroups appended for the LoRA-gradient sum: one per CU the tiles leave idle in
// their last round (the tiles take one CU each; 256 CUs), so the sum runs beside the
// tiles; when that leaves fewer than 16, up to 64 that run as tiles finish. At most one
// output per thread.
int tail_workgroups(int tiles, int64_t items) {
  if (items <= 0) return 0;
  constexpr int NUM_CU = 256;
  const int idle = (NUM_CU - tiles % NUM_CU) % NUM_CU;
  const int64_t need = (items + Waves<GEMM_NWN>::NT - 1) / Waves<GEMM_NWN>::NT;
  const int64_t n = need < (idle >= 16 ? idle : 64) ? need : (idle >= 16 ? idle : 64);
  return (int)(n < 1 ? 1 : n);
}

hipError_t launch_gemm_mx4(const GemmArgs& g, bool trans_b, bool out_bf16, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.Kred < 1 || g.Kred > GEMM_MAX_KRED) return hipErrorInvalidValue;  // the last step is peeled: KT >= 1
  if (g.epi != GEMM_EPI_NONE && (g.epi != GEMM_EPI_DGELU_Q || !out_bf16 || !trans_b || g.q_codes == nullptr ||
                                 g.q_scales == nullptr || g.pre == nullptr))
    return hipErrorInvalidValue;
  const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  if (g.tail.items > 0 && !trans_b) return hipErrorInvalidValue;
  dim3 grid(tiles + tail_workgroups(tiles, g.tail.items)), block(Waves<GEMM_NWN>::NT);
  if (g.epi == GEMM_EPI_DGELU_Q) {
    hipLaunchKernelGGL((k_gemm_mx4<true, true, GEMM_EPI_DGELU_Q, GEMM_NWN>), grid, block, 0, stream, g);
  } else if (!trans_b) {
    if (out_bf16)
      hipLaunchKernelGGL((k_gemm_mx4<false, true, GEMM_EPI_NONE, GEMM_NWN>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_mx4<false, false, GEMM_EPI_NONE, GEMM_NWN>), grid, block, 0, stream, g);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((k_gemm_mx4<true, true, GEMM_EPI_NONE, GEMM_NWN>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_mx4<true, false, GEMM_EPI_NONE, GEMM_NWN>), grid, block, 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace ft
