// Fused quantization + low-rank down-projection (FourTune §3.3 "LoRA Fusion": all
// three branches read the same input, so its quantization and every down-projection
// happen in one kernel and the input is read from HBM once).
//
//   forward : X -> Q(X), XL = bf16( bf16(X) [A; L1]^T )     D rows given (K-contiguous)
//   backward: G -> Q(G), GB = bf16( bf16(G) [B | L2] )       U rows given (rt-contiguous)
//
// HBM-bound: 2 (bf16) or 4 (fp32) bytes read and 0.5 written per input element, plus
// the small [M x rt] output. The down-projection runs on bf16 MFMA 16x16x32. Two
// kernels: bf16 input (every shape the library runs, and the MLP's pass over the saved
// FC1 output with GELU in front) takes the staged kernel further below, which moves
// every operand through LDS; fp32 input takes the register kernel described here,
// which multiplies straight from the registers the quantizer loaded.
//
// Work split. A workgroup of 4 waves owns 64 rows (two block rows) and one of S
// contiguous column ranges; wave w walks the range's 64-column chunks w, w+4, ....
// Register layout of a chunk = the 16x16x32 MFMA operand layout: lane l holds, for
// row group g (rows 16g + l%16) and column block b (32 columns), the 8 values at
// columns 32b + 8(l/16) .. +8 (two 16-byte loads per row, rounded to bf16 for the
// MFMA); a 32x32 quantization block is row groups 2h, 2h+1 of column block b, its
// maximum met over the 64 lanes in VALU exchanges, and the E2M1 conversion is the
// hardware one.
//
// Low-rank side, in 16-wide tiles (ranks are multiples of 16, so tiles never mix the
// two factors). The kernels take the tiles in pairs: a width rank + stab_rank of 16
// (mod 32) runs with one more tile past the second factor, which reads zeros (its
// loads are out of range or masked) and whose output columns are not stored. Forward,
// tile t's rows of [A; L1] are loaded into
// registers in the same layout as the input (they are the MFMA's first operand);
// backward, [B | L2] is rt-contiguous, so each wave stages its chunk's rows in LDS
// with direct-to-LDS loads and reads them transposed (ds_read_b64_tr_b16).
//
// Pipeline. Each wave alternates two register sets (and, backward, two LDS stages):
// chunk i+1 is in flight while chunk i is worked on. Loads into registers are awaited
// by the compiler's own counters; the backward's LDS stages are awaited with exact
// vmcnt counts, which is why every load and store is issued unconditionally (masked
// lanes use out-of-range offsets) and the loop is entered with the same sequence of
// outstanding operations as each later trip.
//
// Reduction. The four waves' fp32 partial products are summed in LDS in wave order.
// With S > 1 each range's sum goes to an fp32 partial buffer and a second kernel adds
// the S partials in range order and rounds once to bf16, so the result does not
// depend on timing. (A last-arriving-workgroup reduction inside this kernel needs
// device-scope fences, which on this chip write back and invalidate the L2 of the
// issuing XCD: measured at 4608 x 3072, the kernel went from 13 to 60 us, against
// ~4.5 us for the second kernel.)
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {

constexpr int QD_WAVES = 4;
constexpr int QD_ROWS = 64;    // rows per workgroup (two block rows, four row groups)
constexpr int CHUNK = 64;      // columns per wave iteration (two blocks)
constexpr int QD_STORES = 12;  // stores per chunk: 8 code words + 4 scale bytes
constexpr int QD_TARGET_WGS = 256;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ v4f mfma16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// fp32 values are kept as float vectors: converting whole vectors (never single int
// lanes bit-cast to float) keeps the compiler's E2M1 conversion operands intact.
struct XChunk {
  static constexpr int LOADS = 16;
  v4f v[4][2][2];
  __device__ void load(bufres r, const uint32_t (&row_off)[4], const bool (&row_ok)[4], int64_t c0, int64_t K,
                       int lq) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t c = c0 + 32 * b + 8 * lq;
        const uint32_t off = sel_off(row_ok[g] && c < K, row_off[g] + (uint32_t)(c * 4));
        v[g][b][0] = __builtin_bit_cast(v4f, buf_load16(r, off));
        v[g][b][1] = __builtin_bit_cast(v4f, buf_load16(r, off + 16));  // OOB + 16 is still OOB
      }
  }
  __device__ uint32_t absmax(int g, int b) const {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const v4i w = __builtin_bit_cast(v4i, v[g][b][q]) & 0x7FFFFFFF;
      m = umax(m, umax(umax((uint32_t)w.x, (uint32_t)w.y), umax((uint32_t)w.z, (uint32_t)w.w)));
    }
    return m;
  }
  __device__ uint32_t codes(int g, int b, float scale) const {
    const v4f x = v[g][b][0], y = v[g][b][1];
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return cvt8_f32(f, scale);
  }
  __device__ v4i operand(int g, int b) const {  // bf16(x), round to nearest even
    const v4f x = v[g][b][0], y = v[g][b][1];
    return v4i{(int)pack_bf16x2(x.x, x.y), (int)pack_bf16x2(x.z, x.w), (int)pack_bf16x2(y.x, y.y),
               (int)pack_bf16x2(y.z, y.w)};
  }
};

// Forward low-rank operand of a chunk: tile t (16 rows j of [A; L1]), column block b,
// in the input's layout. The first `ta` tiles come from d0 (A), the rest from d1 (L1);
// the choice is uniform per tile.
template <int TP>
struct DChunk {
  static constexpr int LOADS = 2 * TP;
  v4i v[TP > 0 ? TP : 1][2];
  __device__ void load(bufres rd0, bufres rd1, int ta, int64_t c0, int64_t K, int lr, int lq) {
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const bool first = t < ta;
      const int64_t j = (first ? 16 * t : 16 * (t - ta)) + lr;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t c = c0 + 32 * b + 8 * lq;
        v[t][b] = buf_load16(first ? rd0 : rd1, sel_off(c < K, (uint32_t)((j * K + c) * 2)));
      }
    }
  }
};

// Backward low-rank stage in LDS: unit q = 8 consecutive j (16 bytes) of the chunk's 64
// rows of [B | L2], row n - c0 at 16*(n - c0); units are QSTRIDE apart (64 bytes of
// padding keep the transposed reads free of bank conflicts).
template <int TP>
struct UStage {
  static constexpr int LOADS = 2 * TP;  // 16-byte direct-to-LDS loads per lane per chunk
  static constexpr int QSTRIDE = 1024 + 64;
  static constexpr int BYTES = 2 * TP * QSTRIDE;
};

template <int TP>
__device__ __forceinline__ void fetch_u(lds_char* sd, bufres rd0, bufres rd1, int ta, int r0, int rt, int64_t c0,
                                        int64_t K, int lane) {
  const int64_t n = c0 + lane;
  const bool nok = n < K;
#pragma unroll
  for (int q = 0; q < 2 * TP; ++q) {
    const bool first = q < 2 * ta;  // uniform
    const int j0 = first ? 8 * q : 8 * (q - 2 * ta);
    const uint32_t off = first ? (uint32_t)((n * r0 + j0) * 2) : (uint32_t)((n * (rt - r0) + j0) * 2);
    // units past the second factor (the padding tile) load zeros, not the next row
    buf_load16_lds(first ? rd0 : rd1, sd + q * UStage<TP>::QSTRIDE, sel_off(nok && (first || j0 < rt - r0), off));
  }
}

// Transposed read of the backward operand, tile t (j = 16t .. +16), column block b:
// lane l receives column j = 16t + l%16 at rows n = 32b + 8(l/16) .. +8 (the
// 16x16x32 MFMA's first operand). Within each 16-lane group, lane s addresses 4
// consecutive j (16t + 4(s%4)) of row n = 32b + 8g + s/4; ds_read_b64_tr_b16 hands
// lane s column 16t + s of those 4 rows, and a second read 64 bytes on covers rows
// +4 .. +8. The reads wait for themselves inside the asm block: the compiler would
// otherwise hold each LDS read back until every direct-to-LDS load in flight
// (including the next chunk's operand) had landed.
__device__ __forceinline__ uint32_t utr_addr(const lds_char* sd, int t, int b, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int j = 16 * t + 4 * (s & 3);
  const int n = 32 * b + 8 * g + (s >> 2);
  return (uint32_t)(uintptr_t)(sd + (j >> 3) * UStage<1>::QSTRIDE + n * 16 + (j & 7) * 2);
}

template <int TP>
__device__ __forceinline__ void lds_tr_tiles(const lds_char* sd, int b, int lane, v4i* out) {
#pragma unroll
  for (int t = 0; t < TP; t += 2) {
    const uint32_t p0 = utr_addr(sd, t, b, lane);
    const uint32_t p1 = utr_addr(sd, t + 1, b, lane);
    v2i w, x, y, z;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:64\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w), "=&v"(x), "=&v"(y), "=&v"(z)
        : "v"(p0), "v"(p1)
        : "memory");
    out[t] = v4i{w.x, w.y, x.x, x.y};
    out[t + 1] = v4i{y.x, y.y, z.x, z.y};
  }
}

// Sum of the 4 waves' [64 x rt] partial products in LDS (wave order), then this column
// range's result: fp32 partials when the range is one of S > 1, else bf16(low). Called
// with every wave's LDS use finished (the area aliases the stages).
template <int TP, int NW = QD_WAVES>
__device__ __forceinline__ void reduce_waves(const v4f (&acc)[4][TP], float* red, const QuantDownArgs& a, int64_t r0,
                                             int split, int S, int wave, int lane, int tid) {
  // acc[g][t] register r of lane l: row 16g + l%16, column 16t + 4(l/16) + r
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int t = 0; t < TP; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((wave * 4 + g) * TP + t) * 4 + r) * 64 + lane] = acc[g][t][r];
  __syncthreads();
  constexpr int NI = 4 * TP * 64;
  const bool partial = S > 1;
  // outputs (and partials) are [M x rt]; a padding tile's columns (>= rt) are dropped
  float* part = a.partials + ((int64_t)split * a.M) * a.rt;
  for (int e = tid; e < NI; e += 64 * NW) {
    const int l = e & 63, t = (e >> 6) % TP, g = e / (64 * TP);
    v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* src = red + ((((w * 4 + g) * TP + t) * 4) * 64 + l);
      s += v4f{src[0], src[64], src[128], src[192]};
    }
    const int64_t orow = r0 + 16 * g + (l & 15);
    const int col = 16 * t + 4 * (l >> 4);
    if (orow < a.M && col < a.rt) {
      if (partial)
        *reinterpret_cast<v4f*>(part + orow * a.rt + col) = s;
      else
        *reinterpret_cast<uint2*>(a.low + orow * a.rt + col) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    }
  }
}

template <int TP, bool UCOLS, int MODE>
__global__ __launch_bounds__(256) void k_quant_down(const QuantDownArgs a) {
  static_assert(TP % 2 == 0, "16-wide low-rank tiles come in pairs");
  static_assert(MODE == QD_QUANT || MODE == QD_DOWN, "quantize + down-projection, or down-projection alone");
  constexpr int NS = MODE == QD_QUANT ? QD_STORES : 0;  // stores per chunk
  constexpr int WAVE_LDS = UCOLS ? 2 * UStage<TP>::BYTES : 0;
  constexpr int RED = QD_WAVES * 4 * TP * 4 * 64 * 4;
  constexpr int SMEM = QD_WAVES * WAVE_LDS > RED ? QD_WAVES * WAVE_LDS : RED;
  constexpr int NX = XChunk::LOADS, NU = UStage<TP>::LOADS;
  __shared__ __align__(16) char smem_raw[SMEM > 0 ? SMEM : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * QD_ROWS;
  const int split = blockIdx.y, S = gridDim.y;
  const int64_t nchunks = (a.K + CHUNK - 1) / CHUNK;
  const int64_t per = (nchunks + S - 1) / S;
  const int64_t ch0 = split * per, ch1 = min(nchunks, ch0 + per);
  const int64_t cpitch = a.K >> 1, nkb = a.K >> 5;
  const int ta = a.r0 / 16;  // tiles of the first factor

  const bufres rx = make_buf(a.x, (uint64_t)a.M * a.ldx * 4);
  const bufres rcodes = make_buf(a.codes, (uint64_t)a.M * cpitch);
  const bufres rscales = make_buf(a.scales, (uint64_t)((a.M + 31) / 32) * nkb);
  uint32_t row_off[4];
  bool row_ok[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t row = r0 + 16 * g + lr;
    row_ok[g] = row < a.M;
    row_off[g] = (uint32_t)(row * a.ldx * 4);
  }
  const bufres rd0 = make_buf(a.d0, (uint64_t)a.K * a.r0 * 2);
  const bufres rd1 = make_buf(a.d1, (uint64_t)a.K * (a.rt - a.r0) * 2);

  v4f acc[4][TP > 0 ? TP : 1];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[g][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // chunks past the range move nothing: their column start is K, so every access is OOB
  auto cstart = [&](int64_t ch) { return ch < ch1 ? ch * CHUNK : a.K; };

  // ---- one chunk: down-projection MFMAs, then the quantization of its four blocks
  auto work = [&](const XChunk& x, const DChunk<TP>& d, const lds_char* sd, int64_t ch) {
    const int64_t c0 = cstart(ch);
    if constexpr (TP > 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        v4i xop[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          xop[g] = x.operand(g, b);
        }
        v4i dop[TP];
        if constexpr (UCOLS) {
          lds_tr_tiles<TP>(sd, b, lane, dop);
        } else {
#pragma unroll
          for (int t = 0; t < TP; ++t) dop[t] = d.v[t][b];
        }
#pragma unroll
        for (int t = 0; t < TP; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) acc[g][t] = mfma16(dop[t], xop[g], acc[g][t]);
      }
    }
    if constexpr (MODE == QD_QUANT)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t bc = c0 + 32 * b;
          const bool bok = bc < a.K;
          const uint32_t amax = wave_max_u32(umax(x.absmax(2 * h, b), x.absmax(2 * h + 1, b)));
          const uint32_t sb = scale_byte_from_amax(amax);
          const float scale = e8m0_to_f32_scale(sb);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int g = 2 * h + q;
            const int64_t row = r0 + 16 * g + lr;
            uint32_t cw = x.codes(g, b, scale);
            if (sb == 0xFFu) cw = 0;
            buf_store4(rcodes, sel_off(bok && row_ok[g], (uint32_t)(row * cpitch + ((bc + 8 * lq) >> 1))), cw);
          }
          buf_store1(rscales,
                     sel_off(bok && lane == 0 && r0 + 32 * h < a.M, (uint32_t)((r0 / 32 + h) * nkb + (bc >> 5))),
                     sb);
        }
  };

  // Two chunks per trip, each in its own register set (and, operand staged in LDS, its
  // own LDS stage); the second may lie past the range: it then loads zeros and stores
  // nothing, which keeps the trip branch-free and its memory-operation count fixed.
  XChunk x0, x1;
  DChunk<TP> d0, d1;
  int64_t ch = ch0 + wave;
  // The empty asm statements with a memory clobber pin the order of the groups of
  // memory operations and the scheduling barriers keep each chunk's arithmetic after
  // the loads issued ahead of it (the scheduler would otherwise hoist it above them
  // and wait for those loads too).
  // Out-of-range stores standing in for a chunk's stores: the loop is entered with the
  // same sequence of outstanding memory operations as each later trip, so the waits
  // (the compiler's for register loads, the explicit ones for the LDS stages) are no
  // stricter than needed.
  auto dummy_stores = [&]() {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      uint32_t off = BUF_OOB + 16u * i;  // distinct, opaque: none may be merged away
      asm volatile("" : "+v"(off));
      buf_store4(rcodes, off, 0u);
    }
  };
  if constexpr (!UCOLS) {
    // Two register sets: while one chunk is worked on, the next chunk's loads are in
    // flight. Both chunks of a trip run; the second may lie past the range (then it
    // loads zeros and stores nothing). The wait before each chunk is the compiler's,
    // counted exactly: the chunk issued after it and one chunk's stores stay in flight.
    x0.load(rx, row_off, row_ok, cstart(ch), a.K, lq);
    d0.load(rd0, rd1, ta, cstart(ch), a.K, lr, lq);
    asm volatile("" ::: "memory");
    dummy_stores();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    for (; ch < ch1; ch += 2 * QD_WAVES) {
      x1.load(rx, row_off, row_ok, cstart(ch + QD_WAVES), a.K, lq);
      d1.load(rd0, rd1, ta, cstart(ch + QD_WAVES), a.K, lr, lq);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      work(x0, d0, nullptr, ch);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      x0.load(rx, row_off, row_ok, cstart(ch + 2 * QD_WAVES), a.K, lq);
      d0.load(rd0, rd1, ta, cstart(ch + 2 * QD_WAVES), a.K, lr, lq);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      work(x1, d1, nullptr, ch + QD_WAVES);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    lds_char* sd0 = (lds_char*)smem_raw + wave * WAVE_LDS;
    lds_char* sd1 = sd0 + UStage<TP>::BYTES;
    auto fetch = [&](lds_char* sd, int64_t c) { fetch_u<TP>(sd, rd0, rd1, ta, a.r0, a.rt, cstart(c), a.K, lane); };
    fetch(sd0, ch);
    asm volatile("" ::: "memory");
    x0.load(rx, row_off, row_ok, cstart(ch), a.K, lq);
    asm volatile("" ::: "memory");
    dummy_stores();
    asm volatile("" ::: "memory");
    fetch(sd1, ch + QD_WAVES);
    wait_vmcnt<NX + NS + NU>();  // operand of chunk ch in sd0
    __builtin_amdgcn_sched_barrier(0);
    for (; ch < ch1; ch += 2 * QD_WAVES) {
      x1.load(rx, row_off, row_ok, cstart(ch + QD_WAVES), a.K, lq);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      work(x0, d0, sd0, ch);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // sd0 reads done before it is refilled
      fetch(sd0, ch + 2 * QD_WAVES);
      wait_vmcnt<NX + NS + NU>();  // operand of chunk ch + 4 in sd1
      __builtin_amdgcn_sched_barrier(0);
      x0.load(rx, row_off, row_ok, cstart(ch + 2 * QD_WAVES), a.K, lq);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      work(x1, d1, sd1, ch + QD_WAVES);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fetch(sd1, ch + 3 * QD_WAVES);
      wait_vmcnt<NX + NS + NU>();  // operand of chunk ch + 8 in sd0
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if constexpr (TP > 0) {
    // ---- sum the 4 waves' partials (LDS), then this range's [64 x rt] result. The
    // backward's stages alias the reduction area: let every direct-to-LDS load land.
    if constexpr (UCOLS) wait_vmcnt<0>();
    __syncthreads();
    reduce_waves<TP>(acc, (float*)smem_raw, a, r0, split, S, wave, lane, tid);
  }
}

// ---------------------------------------------------------------- staged kernel
// bf16 input, rank + stab_rank <= 128. The same work split as k_quant_down (64 rows
// per workgroup, one of S column ranges, 64-column chunks, the same MFMA layouts), but
// every operand reaches LDS by direct-to-LDS loads of whole rows of a chunk and the
// codes leave through LDS, 64 contiguous bytes per row. Measured on the register kernel
// with bf16 input (which it then also served) at 4608 x 3072 (rank + stab_rank = 64):
// without its code stores its loop ran 31% faster, without its X loads or its operand
// loads about a third faster each, without its quantization arithmetic or its MFMAs
// about 5%: the time went to the number of memory requests (a load there spans 16 rows
// x 64 bytes, a code store 16 rows x 16 bytes), not to arithmetic.
//
// 8 waves, two per SIMD, each on its own LDS area with no barrier until the final
// reduction: one stage (one chunk of X and of the low-rank operand) and a code buffer
// for two chunks. While one wave of a SIMD waits for its chunk, the other converts and
// quantizes (with one wave per SIMD and two stages each, those waits and the vector
// arithmetic added up: at K = 12288 a chunk took 1.03 us without quantization, 1.66 us
// with it and 3.1 us with GELU in front; two waves per SIMD took the GELU pass from 55
// to 45 us). A wave takes its chunks in adjacent pairs (chunks 2w, 2w+1 of every 16), so
// the codes of a pair are 64 contiguous bytes of each row, and works on a chunk in two
// halves (column blocks b = 0, 1) so that it fits the 256 registers two waves per SIMD
// leave it. Layouts:
//   X, and D in the forward: chunk row r at 128 r, its 16-byte unit u at slot
//     u ^ ((r >> 1) & 7) (the 16 rows an operand read touches meet 16 bank groups);
//   backward: the chunk's 64 rows of each factor of [B | L2] contiguous as in memory
//     (row pitch 2 r_f bytes; first factor, then second), read transposed;
//   codes: row r at 64 r, unit u at slot u ^ ((r >> 2) & 3).
// Loads are awaited with exact vmcnt counts (every load and store is issued, dead ones
// at out-of-range offsets), and all LDS accesses inside the loop are written in asm
// that waits for itself: the compiler, seeing direct-to-LDS loads into the same array,
// would otherwise wait for all of them before every LDS access.
constexpr int SQ_XB = QD_ROWS * 128;  // X per stage: 64 rows x 64 bf16
constexpr int SQ_CB = QD_ROWS * 64;   // codes of two chunks: 64 rows x 64 bytes
__device__ __forceinline__ int sq_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// 16-byte LDS reads (four or two), awaited inside the block.
__device__ __forceinline__ void lds_read16x4(const uint32_t (&ad)[4], v4i (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
}
__device__ __forceinline__ void lds_read16x2(const uint32_t (&ad)[2], v4i (&o)[2]) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1])
               : "v"(ad[0]), "v"(ad[1])
               : "memory");
}

// Waves per workgroup: 8 (two per SIMD) up to four low-rank tiles. With six or eight,
// a wave's accumulators and operand tiles need more than the 256 registers two waves
// per SIMD leave it (six waves spilled 35-82 registers), so 4 waves run, one per SIMD.
template <int TP>
constexpr int sq_waves() { return TP <= 4 ? 8 : 4; }
// LDS of the staged kernel: per wave one stage (X chunk, low-rank operand chunk) and the
// code buffer; after the loop the same bytes hold the waves' partial products.
template <int TP>
struct SqLds {
  static constexpr int NW = sq_waves<TP>();
  static constexpr int DB = 2048 * TP;  // low-rank operand per stage: 16 TP x 64 bf16
  static constexpr int STAGE = SQ_XB + DB;
  static constexpr int WAVE = STAGE + SQ_CB;
  static constexpr int RED = NW * 4 * TP * 4 * 64 * 4;
  static constexpr int BYTES = NW * WAVE > RED ? NW * WAVE : RED;
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// The low-rank operand of column block b (32 columns) of a staged chunk at sd, as the
// 16x16x32 MFMA's first operand: dv[t] = tile t (16 low-rank columns). Forward layout:
// [A; L1] rows jj at 128 jj, unit u at slot u ^ sq_swz(jj). Backward layout: the chunk's
// 64 rows of each factor of [B | L2] as in memory (row pitch 2 r_f bytes; first factor,
// then second), read transposed with ds_read_b64_tr_b16. A padding tile (16t >= rt)
// reads in range and is zeroed. The reads wait for themselves (see the kernels' notes
// on direct-to-LDS loads).
template <int TP, bool UCOLS>
__device__ __forceinline__ void read_lowrank(const lds_char* const sd, int b, int lane, int ta, int r0, int r1, int rt,
                                             v4i (&dv)[TP]) {
  const int lr = lane & 15, lq = lane >> 4;
  if constexpr (!UCOLS) {
    uint32_t ad[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const int jj = 16 * t + lr;
      ad[t] = lds_addr(sd + jj * 128 + (((4 * b + lq) ^ sq_swz(jj)) << 4));
    }
#pragma unroll
    for (int t0 = 0; t0 < TP; t0 += 4) {
      if constexpr (TP % 4 == 0) {
        lds_read16x4(*reinterpret_cast<const uint32_t(*)[4]>(ad + t0), *reinterpret_cast<v4i(*)[4]>(dv + t0));
      } else if (t0 + 4 <= TP) {
        lds_read16x4(*reinterpret_cast<const uint32_t(*)[4]>(ad + t0), *reinterpret_cast<v4i(*)[4]>(dv + t0));
      } else {
        lds_read16x2(*reinterpret_cast<const uint32_t(*)[2]>(ad + t0), *reinterpret_cast<v4i(*)[2]>(dv + t0));
      }
    }
  } else {
    const int gq = lane >> 4, s = lane & 15;
#pragma unroll
    for (int t = 0; t < TP; t += 2) {
      uint32_t p[2], pitch[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool first = t + u < ta;
        const int rf = first ? r0 : r1;
        const int jl = 16 * (first ? t + u : t + u - ta) + 4 * (s & 3);
        const int n = 32 * b + 8 * gq + (s >> 2);
        pitch[u] = (uint32_t)(2 * rf);
        p[u] = lds_addr(sd + (first ? 0 : 128 * r0)) + (uint32_t)(n * 2 * rf + 2 * jl);
        if (16 * (t + u) >= rt) p[u] = lds_addr(sd), pitch[u] = 0;  // padding tile: read in range, zeroed below
      }
      v2i w, x, y, z;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %5\n\t"
          "ds_read_b64_tr_b16 %2, %6\n\t"
          "ds_read_b64_tr_b16 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(w), "=&v"(x), "=&v"(y), "=&v"(z)
          : "v"(p[0]), "v"(p[0] + 4 * pitch[0]), "v"(p[1]), "v"(p[1] + 4 * pitch[1])
          : "memory");
      dv[t] = v4i{w.x, w.y, x.x, x.y};
      dv[t + 1] = v4i{y.x, y.y, z.x, z.y};
      if (16 * t >= rt) dv[t] = v4i{0, 0, 0, 0};
      if (16 * (t + 1) >= rt) dv[t + 1] = v4i{0, 0, 0, 0};
    }
  }
}

template <int TP, bool UCOLS, int MODE>
__global__ __launch_bounds__(64 * sq_waves<TP>()) void k_quant_down_lds(const QuantDownArgs a) {
  static_assert(TP % 2 == 0 && TP <= 8, "staged kernel: rank + stab_rank <= 128");
  constexpr int NW = sq_waves<TP>();
  using L = SqLds<TP>;
  constexpr bool QUANT = MODE == QD_QUANT || MODE == QD_GELU_QUANT;
  constexpr int NS = QUANT ? 5 : 0;  // stores per pair: 4 code blocks, 1 scale
  __shared__ __align__(16) char smem_raw[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * QD_ROWS;
  const int rows_left = (int)min<int64_t>(a.M - r0, QD_ROWS);
  const int split = blockIdx.y, S = gridDim.y;
  const int64_t nchunks = (a.K + CHUNK - 1) / CHUNK;
  const int64_t per = (nchunks + S - 1) / S;
  const int64_t ch0 = split * per, ch1 = min(nchunks, ch0 + per);
  const int rounds = (int)((max<int64_t>(ch1 - ch0, 0) + 2 * NW - 1) / (2 * NW));
  const int64_t cpitch = a.K >> 1, nkb = a.K >> 5;
  const int ta = a.r0 / 16, r1 = a.rt - a.r0;

  const bufres rx = make_buf(a.x, (uint64_t)a.M * a.ldx * 2);
  const bufres rcodes = make_buf(a.codes, (uint64_t)a.M * cpitch);
  const bufres rscales = make_buf(a.scales, (uint64_t)((a.M + 31) / 32) * nkb);
  const bufres rd0 = make_buf(a.d0, (uint64_t)a.K * a.r0 * 2);
  const bufres rd1 = make_buf(a.d1, (uint64_t)a.K * r1 * 2);

  lds_char* const st = (lds_char*)smem_raw + wave * L::WAVE;
  lds_char* const cbuf = st + L::STAGE;

  v4f acc[4][TP > 0 ? TP : 1];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int t = 0; t < (TP > 0 ? TP : 1); ++t) acc[g][t] = v4f{0.f, 0.f, 0.f, 0.f};

  auto chunk_of = [&](int k, int i) -> int64_t { return ch0 + 2 * NW * k + 2 * wave + i; };

  auto dma = [&](int64_t c) __attribute__((always_inline)) {
    const bool live = c < ch1;
    const int64_t c0 = c * CHUNK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int64_t col = c0 + 8 * ((lane & 7) ^ sq_swz(row));
      buf_load16_lds(rx, st + i * 1024,
                     sel_off(live && row < rows_left && col < a.K, (uint32_t)(((r0 + row) * a.ldx + col) * 2)));
    }
    if constexpr (TP > 0) {
      lds_char* const sd = st + SQ_XB;
#pragma unroll
      for (int i = 0; i < 2 * TP; ++i) {
        const bool first = 8 * i < a.r0;
        if constexpr (!UCOLS) {
          const int jj = 8 * i + (lane >> 3);
          const int64_t j = first ? jj : jj - a.r0;
          const int64_t col = c0 + 8 * ((lane & 7) ^ sq_swz(jj));
          buf_load16_lds(first ? rd0 : rd1, sd + i * 1024, sel_off(live && col < a.K, (uint32_t)((j * a.K + col) * 2)));
        } else {
          const int rf = first ? a.r0 : r1;
          const int o = (first ? i : i - a.r0 / 8) * 1024 + 16 * lane;
          // the chunk's rows of a factor are 128 rf bytes; past them (the padding tile)
          // nothing is loaded
          const bool ok = live && (int64_t)o < (a.K - c0) * 2 * rf && o < 128 * rf;
          buf_load16_lds(first ? rd0 : rd1, sd + i * 1024, sel_off(ok, (uint32_t)(c0 * 2 * rf + o)));
        }
      }
    }
  };

  uint32_t sbs0 = 0, sbs1 = 0;
  // column block b (32 columns) of chunk i (0, 1) of the pair. The second block's last
  // read of the stage is followed by the loads of chunk `pf` into it, which then land
  // while that block's arithmetic runs.
  auto work_half = [&](int i, int b, int64_t cc, int64_t pf) __attribute__((always_inline)) {
    v4i xv[4];  // rows 16g + l%16, columns 32b + 8(l/16) .. +8
    {
      uint32_t ad[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = 16 * g + lr;
        ad[g] = lds_addr(st + row * 128 + (((4 * b + lq) ^ sq_swz(row)) << 4));
      }
      lds_read16x4(ad, xv);
    }
    if constexpr (TP == 0) {
      if (b == 1) dma(pf);
    }
    float hv[4][8];
    if constexpr (MODE == QD_GELU_QUANT) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t ws[4] = {(uint32_t)xv[g].x, (uint32_t)xv[g].y, (uint32_t)xv[g].z, (uint32_t)xv[g].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[g][2 * e] = gelu_f(bf16_lo(ws[e]));
          hv[g][2 * e + 1] = gelu_f(bf16_hi(ws[e]));
        }
      }
      // optional export of the fp32 H that Q(H) quantizes. These stores precede the
      // pair's code stores, so the exact vmcnt waits below stay correct (operations
      // complete in issue order; extra ones ahead of the last NS only make a wait
      // stricter).
      if (a.hdbg != nullptr) {
        const bufres rh = make_buf(a.hdbg, (uint64_t)a.M * a.K * 4);
        const int64_t col = cc * CHUNK + 32 * b + 8 * lq;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t row = r0 + 16 * g + lr;
          const uint32_t off = sel_off(cc < ch1 && row < a.M && col < a.K, (uint32_t)((row * a.K + col) * 4));
          buf_store16(rh, off, __builtin_bit_cast(v4i, v4f{hv[g][0], hv[g][1], hv[g][2], hv[g][3]}));
          buf_store16(rh, off + 16, __builtin_bit_cast(v4i, v4f{hv[g][4], hv[g][5], hv[g][6], hv[g][7]}));
        }
      }
    }
    if constexpr (TP > 0) {
      v4i dv[TP];
      read_lowrank<TP, UCOLS>(st + SQ_XB, b, lane, ta, a.r0, r1, a.rt, dv);
      if (b == 1) dma(pf);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v4i xop;
        if constexpr (MODE == QD_GELU_QUANT)
          xop = v4i{(int)pack_bf16x2(hv[g][0], hv[g][1]), (int)pack_bf16x2(hv[g][2], hv[g][3]),
                    (int)pack_bf16x2(hv[g][4], hv[g][5]), (int)pack_bf16x2(hv[g][6], hv[g][7])};
        else
          xop = xv[g];
#pragma unroll
        for (int t = 0; t < TP; ++t) acc[g][t] = mfma16(dv[t], xop, acc[g][t]);
      }
    }
    if constexpr (QUANT) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int g = 2 * h + q;
          if constexpr (MODE == QD_GELU_QUANT) {
#pragma unroll
            for (int e = 0; e < 8; ++e) m = umax(m, __builtin_bit_cast(uint32_t, hv[g][e]) & 0x7FFFFFFFu);
          } else {
            const v4i w = xv[g];
            m = umax(m, umax(umax(bf16x2_absmax_bits(w.x), bf16x2_absmax_bits(w.y)),
                             umax(bf16x2_absmax_bits(w.z), bf16x2_absmax_bits(w.w))));
          }
        }
        const uint32_t sb = scale_byte_from_amax(wave_max_u32(m));
        const float scale = e8m0_to_f32_scale(sb);
        if (h == 0) sbs0 |= sb << (8 * (2 * i + b));
        else sbs1 |= sb << (8 * (2 * i + b));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int g = 2 * h + q;
          uint32_t cw;
          if constexpr (MODE == QD_GELU_QUANT) {
            cw = cvt8_f32(hv[g], scale);
          } else {
            const v4i w = xv[g];
            cw = cvt8_bf16(w.x, w.y, w.z, w.w, scale);
          }
          if (sb == 0xFFu) cw = 0;
          const int row = 16 * g + lr;
          const uint32_t ad = lds_addr(cbuf + row * 64 + (((2 * i + b) ^ ((row >> 2) & 3)) << 4) + 4 * lq);
          asm volatile("ds_write_b32 %0, %1" ::"v"(ad), "v"(cw) : "memory");
        }
      }
    }
  };
  auto work = [&](int i, int64_t cc, int64_t pf) __attribute__((always_inline)) {
    work_half(i, 0, cc, pf);
    work_half(i, 1, cc, pf);
  };

  auto store_pair = [&](int k) __attribute__((always_inline)) {
    const int64_t pc = chunk_of(k, 0) * CHUNK;
    uint32_t ad[4];
    v4i cv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * q + (lane >> 2), u = lane & 3;
      ad[q] = lds_addr(cbuf + row * 64 + ((u ^ ((row >> 2) & 3)) << 4));
    }
    lds_read16x4(ad, cv);
    const int u = lane & 3;
    const bool uok = chunk_of(k, u >> 1) < ch1 && pc + 32 * u < a.K;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * q + (lane >> 2);
      buf_store16(rcodes, sel_off(uok && row < rows_left, (uint32_t)((r0 + row) * cpitch + (pc >> 1) + 16 * u)), cv[q]);
    }
    const int h = (lane >> 2) & 1, e = lane & 3;
    const uint32_t v = ((h ? sbs1 : sbs0) >> (8 * e)) & 0xFFu;
    const bool sok = lane < 8 && r0 + 32 * h < a.M && chunk_of(k, e >> 1) < ch1 && pc + 32 * e < a.K;
    buf_store1(rscales, sel_off(sok, (uint32_t)((r0 / 32 + h) * nkb + (pc >> 5) + e)), v);
  };

  dma(chunk_of(0, 0));
  if constexpr (NS > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      uint32_t off = BUF_OOB + 16u * i;
      asm volatile("" : "+v"(off));
      buf_store4(rcodes, off, 0u);
    }
  }
  for (int k = 0; k < rounds; ++k) {
    sbs0 = sbs1 = 0;
    wait_vmcnt<NS>();  // chunk (k, 0) landed; the last pair's stores may still be in flight
    work(0, chunk_of(k, 0), chunk_of(k, 1));
    wait_vmcnt<0>();
    work(1, chunk_of(k, 1), chunk_of(k + 1, 0));
    if constexpr (NS > 0) store_pair(k);
  }
  if constexpr (TP > 0) {
    wait_vmcnt<0>();
    __syncthreads();
    reduce_waves<TP, NW>(acc, (float*)smem_raw, a, r0, split, S, wave, lane, tid);
  }
}

// ---------------------------------------------------------------- row-split kernel
// bf16 input with a wide low-rank operand (rank + stab_rank above 64) over many rows.
// The staged kernel above gives each wave its own chunk and its own copy of that chunk's
// low-rank operand: at rank + stab_rank = 128 a wave's stage is 8 KB of X and 16 KB of
// operand, one stage per wave fits, and a CU has about 32 KB of X in flight. At
// 32760 x 5120 that ran at 38% of HBM while the quantizer alone reached 73%: with a
// latency of ~3 us under full load, 256 CUs x 32 KB in flight is ~2.8 TB/s.
//
// The low-rank operand is read K-contiguous, as [A; L1] is stored; the backward's
// [B | L2] is transposed into that layout first (launch_quant_down).
//
// Here a workgroup owns 128 rows and works on one chunk at a time, all waves together.
// The chunk's X rows and its low-rank operand pass through a ring of four stages shared
// by the workgroup, so three chunks (48 KB of X) are in flight and the operand is
// fetched once per 128 rows instead of once per 64. 8 waves, two per SIMD: waves w and
// w + 4 own rows 32(w%4) .. +32 (one block row), wave w the first 32-column block of
// every chunk and w + 4 the second, so each still quantizes whole 32x32 blocks, and each
// keeps its partial [32 x rt] sums to the end, where the pair's two meet once in LDS.
// With one wave per SIMD (4 waves of 32 rows, both blocks each) the vector work (GELU,
// block maxima, conversions) did not overlap the loads: the MLP's pass over P^ at
// 32760 x 13824 took 414 us against 370 with two. Each chunk costs one workgroup
// barrier. At 32760 x 5120 the kernel moves 52-54% of 8 TB/s; X in registers instead of
// LDS, with more chunks in flight, was slower there: the limit is not the depth of the
// load pipeline.
//
// Waits. Every wave issues, per chunk, its loads of the chunk three ahead (at
// out-of-range offsets past the column range), and after every even chunk's loads the
// stores of the pair before (its codes are complete once both waves of the row group
// have passed the barrier; the code buffer alternates between pairs). The count of a
// wave's own operations issued after a chunk's loads is thus fixed by the chunk's
// parity; the wait before a chunk leaves exactly those in flight, and the barrier after
// it makes every wave's loads of the chunk visible. The loads into a stage are issued
// only after the barrier that follows every wave's last read of it. LDS accesses in the
// loop are asm that waits for itself, as in the staged kernel.
constexpr int QR_ROWS = 128;
constexpr int QR_WAVES = 8;   // two per SIMD
constexpr int QR_STAGES = 4;
#ifndef QR_MIN_M
#define QR_MIN_M 4096
#endif
template <int TP>
struct QrLds {
  static constexpr int XB = QR_ROWS * 128;  // X per stage: 128 rows x 64 bf16
  static constexpr int DB = 16 * 1024;      // low-rank operand per stage: up to 128 rows x 64 bf16
  static constexpr int STAGE = XB + DB;
  static constexpr int CB = 32 * 64;        // codes of a chunk pair for 32 rows, 64 bytes each
  // stages, then the code buffers: [pair parity][row group of waves]
  static constexpr int BYTES = QR_STAGES * STAGE + 2 * 4 * CB;
  static constexpr int RED = 4 * 2 * TP * 64 * 16;  // the second column block's partial sums
  static_assert(BYTES <= 160 * 1024 && RED <= QR_STAGES * STAGE, "LDS");
};

__device__ __forceinline__ v4i lds_read16(uint32_t ad) {
  v4i o;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(o) : "v"(ad) : "memory");
  return o;
}

template <int TP, int MODE>
__global__ __launch_bounds__(64 * QR_WAVES) void k_quant_down_rows(const QuantDownArgs a) {
  static_assert(TP % 2 == 0 && TP >= 2 && TP <= 8, "row-split kernel: 2 .. 8 low-rank tiles (launched with 6, 8)");
  using L = QrLds<TP>;
  constexpr bool QUANT = MODE == QD_QUANT || MODE == QD_GELU_QUANT;
  constexpr int NS = QUANT ? 2 : 0;     // stores per chunk pair and wave: a code piece, the scale bytes
  constexpr int NL = 4;                 // direct-to-LDS loads per chunk and wave: 2 of X, 2 of the operand
  constexpr int AHEAD = QR_STAGES - 1;  // chunks in flight
  // operations a wave issues after a chunk's loads until that chunk is worked on: the
  // loads of the AHEAD - 1 chunks after it, and the stores of the even chunks among the
  // AHEAD from the chunk's issue on (a pair's stores follow its next chunk's loads)
  constexpr int WAIT_EVEN = (AHEAD - 1) * NL + NS * (AHEAD / 2);
  constexpr int WAIT_ODD = (AHEAD - 1) * NL + NS * ((AHEAD + 1) / 2);
  static_assert(WAIT_EVEN < 64 && WAIT_ODD < 64, "vmcnt field");
  __shared__ __align__(16) char smem_raw[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave & 3, bsel = wave >> 2;  // row group of 32, column block of each chunk
  const int lr = lane & 15, lq = lane >> 4;
  const int wrow = 32 * rw;  // this wave's first row in the stripe
  const int64_t r0 = (int64_t)blockIdx.x * QR_ROWS;
  const int rows_left = (int)min<int64_t>(a.M - r0, QR_ROWS);
  const int split = blockIdx.y, S = gridDim.y;
  const int64_t nchunks = (a.K + CHUNK - 1) / CHUNK;
  const int64_t per = (nchunks + S - 1) / S;
  const int64_t ch0 = split * per, ch1 = min(nchunks, ch0 + per);
  const int trips = (int)((max<int64_t>(ch1 - ch0, 0) + 1) / 2);
  const int64_t cpitch = a.K >> 1, nkb = a.K >> 5;
  const int ta = a.r0 / 16, r1 = a.rt - a.r0;

  const bufres rx = make_buf(a.x, (uint64_t)a.M * a.ldx * 2);
  const bufres rcodes = make_buf(a.codes, (uint64_t)a.M * cpitch);
  const bufres rscales = make_buf(a.scales, (uint64_t)((a.M + 31) / 32) * nkb);
  const bufres rd0 = make_buf(a.d0, (uint64_t)a.K * a.r0 * 2);
  const bufres rd1 = make_buf(a.d1, (uint64_t)a.K * r1 * 2);

  lds_char* const stages = (lds_char*)smem_raw;
  lds_char* const codes_lds = stages + QR_STAGES * L::STAGE;
  auto cbuf = [&](int pair) { return codes_lds + ((pair & 1) * 4 + rw) * L::CB; };

  v4f acc[2][TP];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[g][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // loads of local chunk j (column chunk ch0 + j) into stage j % QR_STAGES, pieces
  // 2 wave and 2 wave + 1 of each: X rows 16 wave .. +16, and operand rows 16 wave .. +16
  // (rows past 16 TP, and past the second factor, read as zeros and are never used)
  auto dma = [&](int j) __attribute__((always_inline)) {
    const int64_t c = ch0 + j;
    const bool live = c < ch1;
    const int64_t c0 = c * CHUNK;
    lds_char* const st = stages + (j % QR_STAGES) * L::STAGE;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = 2 * wave + q;
      const int row = 8 * i + (lane >> 3);
      const int64_t col = c0 + 8 * ((lane & 7) ^ sq_swz(row));
      buf_load16_lds(rx, st + i * 1024,
                     sel_off(live & (row < rows_left) & (col < a.K), (uint32_t)(((r0 + row) * a.ldx + col) * 2)));
    }
    lds_char* const sd = st + L::XB;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = 2 * wave + q;
      const bool first = 8 * i < a.r0;
      const int jj = 8 * i + (lane >> 3);
      const int64_t jr = first ? jj : jj - a.r0;
      const int64_t col = c0 + 8 * ((lane & 7) ^ sq_swz(jj));
      buf_load16_lds(first ? rd0 : rd1, sd + i * 1024, sel_off(live & (col < a.K), (uint32_t)((jr * a.K + col) * 2)));
    }
  };
  auto dummy_stores = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      uint32_t off = BUF_OOB + 16u * i;  // distinct, opaque: none may be merged away
      asm volatile("" : "+v"(off));
      buf_store4(rcodes, off, 0u);
    }
  };

  uint32_t sbs = 0;  // this wave's two scale bytes of the current pair (chunk 0, chunk 1)
  // local chunk j, position i (0, 1) in its pair: this wave's column block of it
  auto work = [&](int i, int j) __attribute__((always_inline)) {
    const lds_char* const st = stages + (j % QR_STAGES) * L::STAGE;
    const int64_t cc = ch0 + j;
    const int b = bsel;
    v4i xv[2];  // rows wrow + 16g + l%16, columns 32b + 8(l/16) .. +8
    {
      uint32_t ad[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int row = wrow + 16 * g + lr;
        ad[g] = lds_addr(st + row * 128 + (((4 * b + lq) ^ sq_swz(row)) << 4));
      }
      lds_read16x2(ad, xv);
    }
    float hv[2][8];
    if constexpr (MODE == QD_GELU_QUANT) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t ws[4] = {(uint32_t)xv[g].x, (uint32_t)xv[g].y, (uint32_t)xv[g].z, (uint32_t)xv[g].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[g][2 * e] = gelu_f(bf16_lo(ws[e]));
          hv[g][2 * e + 1] = gelu_f(bf16_hi(ws[e]));
        }
      }
      // optional export of the fp32 H that Q(H) quantizes: extra operations ahead of
      // the pair's stores only make the waits stricter
      if (a.hdbg != nullptr) {
        const bufres rh = make_buf(a.hdbg, (uint64_t)a.M * a.K * 4);
        const int64_t col = cc * CHUNK + 32 * b + 8 * lq;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int64_t row = r0 + wrow + 16 * g + lr;
          const uint32_t off = sel_off(cc < ch1 && row < a.M && col < a.K, (uint32_t)((row * a.K + col) * 4));
          buf_store16(rh, off, __builtin_bit_cast(v4i, v4f{hv[g][0], hv[g][1], hv[g][2], hv[g][3]}));
          buf_store16(rh, off + 16, __builtin_bit_cast(v4i, v4f{hv[g][4], hv[g][5], hv[g][6], hv[g][7]}));
        }
      }
    }
    v4i dv[TP];
    read_lowrank<TP, false>(st + L::XB, b, lane, ta, a.r0, r1, a.rt, dv);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      v4i xop;
      if constexpr (MODE == QD_GELU_QUANT)
        xop = v4i{(int)pack_bf16x2(hv[g][0], hv[g][1]), (int)pack_bf16x2(hv[g][2], hv[g][3]),
                  (int)pack_bf16x2(hv[g][4], hv[g][5]), (int)pack_bf16x2(hv[g][6], hv[g][7])};
      else
        xop = xv[g];
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[g][t] = mfma16(dv[t], xop, acc[g][t]);
    }
    if constexpr (QUANT) {
      uint32_t m = 0;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if constexpr (MODE == QD_GELU_QUANT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) m = umax(m, __builtin_bit_cast(uint32_t, hv[g][e]) & 0x7FFFFFFFu);
        } else {
          const v4i w = xv[g];
          m = umax(m, umax(umax(bf16x2_absmax_bits(w.x), bf16x2_absmax_bits(w.y)),
                           umax(bf16x2_absmax_bits(w.z), bf16x2_absmax_bits(w.w))));
        }
      }
      const uint32_t sb = scale_byte_from_amax(wave_max_u32(m));
      const float scale = e8m0_to_f32_scale(sb);
      sbs = i == 0 ? sb : (sbs | (sb << 8));
      lds_char* const cb = cbuf(j >> 1);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t cw;
        if constexpr (MODE == QD_GELU_QUANT) {
          cw = cvt8_f32(hv[g], scale);
        } else {
          const v4i w = xv[g];
          cw = cvt8_bf16(w.x, w.y, w.z, w.w, scale);
        }
        if (sb == 0xFFu) cw = 0;
        const int row = 16 * g + lr;
        const uint32_t ad = lds_addr(cb + row * 64 + (((2 * i + b) ^ ((row >> 2) & 3)) << 4) + 4 * lq);
        asm volatile("ds_write_b32 %0, %1" ::"v"(ad), "v"(cw) : "memory");
      }
    }
  };

  // codes of pair k (both waves of the row group wrote them before the last barrier):
  // this wave stores rows 16 bsel .. +16 of the group, 64 contiguous bytes each, and its
  // own two scale bytes (blocks bsel and 2 + bsel of the pair's four)
  auto store_pair = [&](int k) __attribute__((always_inline)) {
    const int64_t pc = (ch0 + 2 * k) * CHUNK;
    const int row = 16 * bsel + (lane >> 2), u = lane & 3;
    const v4i cv = lds_read16(lds_addr(cbuf(k) + row * 64 + ((u ^ ((row >> 2) & 3)) << 4)));
    const bool uok = ch0 + 2 * k + (u >> 1) < ch1 && pc + 32 * u < a.K;
    buf_store16(rcodes,
                sel_off(uok && wrow + row < rows_left, (uint32_t)((r0 + wrow + row) * cpitch + (pc >> 1) + 16 * u)),
                cv);
    const int e = 2 * (lane & 1) + bsel;  // lanes 0, 1: chunk 0, 1 of the pair
    const uint32_t v = (sbs >> (8 * (lane & 1))) & 0xFFu;
    const bool sok = lane < 2 && r0 + wrow < a.M && ch0 + 2 * k + (lane & 1) < ch1 && pc + 32 * e < a.K;
    buf_store1(rscales, sel_off(sok, (uint32_t)(((r0 + wrow) / 32) * nkb + (pc >> 5) + e)), v);
  };

  // the issue sequence of the AHEAD chunks before the first: as if issued by chunks
  // -AHEAD .. -1, the even ones of which are followed by a pair's stores
#pragma unroll
  for (int j = 0; j < AHEAD; ++j) {
    dma(j);
    if constexpr (NS > 0)
      if (((j - AHEAD) & 1) == 0) dummy_stores();
  }
  for (int k = 0; k < trips; ++k) {
    wait_vmcnt<WAIT_EVEN>();  // this wave's loads of chunk 2k landed
    // and every wave's (the barrier); the stage of chunk 2k - 1 is read and the codes
    // of pair k - 1 written
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dma(2 * k + AHEAD);
    if constexpr (NS > 0) {
      if (k == 0) dummy_stores();
      else store_pair(k - 1);
    }
    work(0, 2 * k);
    wait_vmcnt<WAIT_ODD>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dma(2 * k + 1 + AHEAD);
    work(1, 2 * k + 1);
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (NS > 0)
    if (trips > 0) store_pair(trips - 1);

  // the row group's [32 x rt] result: the second column block's sums meet the first's
  // in LDS (the stages are free), then bf16 once, or this range's fp32 partial
  // acc[g][t] register r of lane l: row wrow + 16g + l%16, column 16t + 4(l/16) + r
  v4f* red = reinterpret_cast<v4f*>(smem_raw);
  if (bsel == 1) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < TP; ++t) red[((rw * 2 + g) * TP + t) * 64 + lane] = acc[g][t];
  }
  __syncthreads();
  if (bsel == 1) return;
  float* part = a.partials + ((int64_t)split * a.M) * a.rt;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const v4f v = acc[g][t] + red[((rw * 2 + g) * TP + t) * 64 + lane];
      const int64_t orow = r0 + wrow + 16 * g + lr;
      const int col = 16 * t + 4 * lq;
      if (orow < a.M && col < a.rt) {
        if (S > 1)
          *reinterpret_cast<v4f*>(part + orow * a.rt + col) = v;
        else
          *reinterpret_cast<uint2*>(a.low + orow * a.rt + col) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      }
    }
}

// Sum of the S column-range partials of each row, in range order, rounded once to
// bf16.
__global__ __launch_bounds__(256) void k_sum_partials(const float* __restrict__ partials, int S, int64_t n4,
                                                      bf16_t* __restrict__ low) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one v4f of [M x rt]
  if (i >= n4) return;
  const v4f s = sum_ranges(reinterpret_cast<const v4f*>(partials) + i, S, n4);
  *reinterpret_cast<uint2*>(low + 4 * i) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
}

// [B | L2] (K rows: r0 values of the first factor, then r1 of the second, each factor
// row-major) transposed into ut [rt x K]: row j < r0 is column j of the first factor,
// row r0 + j column j of the second. A thread moves one 8 x 8 block: eight 16-byte
// loads (8 rows of the input, 8 consecutive columns each), the transpose in registers,
// eight 16-byte stores; consecutive threads take consecutive column blocks, so each
// input row is read in whole. Ranks are multiples of 16 and K of 32, so a block never
// straddles the two factors or the end of a row.
__device__ __forceinline__ uint32_t pick16(uint32_t lo_src, uint32_t hi_src, bool high) {
  return high ? (lo_src >> 16) | (hi_src & 0xFFFF0000u) : (lo_src & 0xFFFFu) | (hi_src << 16);
}
__global__ __launch_bounds__(256) void k_transpose_u(const bf16_t* __restrict__ d0, const bf16_t* __restrict__ d1,
                                                     int r0, int r1, int64_t K, bf16_t* __restrict__ ut) {
  const int jbs = (r0 + r1) / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (K / 8) * jbs) return;
  const int jb = (int)(t % jbs);
  const int64_t n0 = 8 * (t / jbs);
  const int j0 = 8 * jb;
  const bool first = j0 < r0;
  const bf16_t* src = first ? d0 + j0 : d1 + (j0 - r0);
  const int64_t ld = first ? r0 : r1;
  v4i a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const v4i*>(src + (n0 + i) * ld);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int w = jj >> 1;
    const bool high = jj & 1;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pick16((uint32_t)a[2 * q][w], (uint32_t)a[2 * q + 1][w], high);
    *reinterpret_cast<v4i*>(ut + (int64_t)(j0 + jj) * K + n0) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  }
}

template <bool UCOLS, int MODE>
hipError_t launch_reg(const QuantDownArgs& a, int tp, int splits, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + QD_ROWS - 1) / QD_ROWS), (unsigned)splits), block(256);
  switch (tp) {
    case 0: hipLaunchKernelGGL((k_quant_down<0, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_quant_down<2, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_quant_down<4, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((k_quant_down<6, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_quant_down<8, UCOLS, MODE>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_rows(const QuantDownArgs& a, int tp, int splits, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + QR_ROWS - 1) / QR_ROWS), (unsigned)splits), block(64 * QR_WAVES);
  switch (tp) {
    case 6: hipLaunchKernelGGL((k_quant_down_rows<6, MODE>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_quant_down_rows<8, MODE>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The row-split kernel serves widths above 64 (six or eight 16-wide tiles) from 4096
// rows. At width 64 the staged kernel stays ahead (4608 x 3072: 14.2 against 14.5 us),
// and below 4096 rows its 64-row stripes give more workgroups.
bool use_rows_kernel(int64_t M, int rt) { return rt > 64 && M >= QR_MIN_M; }

template <bool UCOLS, int MODE>
hipError_t launch_staged(const QuantDownArgs& a, int tp, int splits, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + QD_ROWS - 1) / QD_ROWS), (unsigned)splits);
  switch (tp) {
    case 0: hipLaunchKernelGGL((k_quant_down_lds<0, UCOLS, MODE>), grid, dim3(64 * sq_waves<0>()), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_quant_down_lds<2, UCOLS, MODE>), grid, dim3(64 * sq_waves<2>()), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_quant_down_lds<4, UCOLS, MODE>), grid, dim3(64 * sq_waves<4>()), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((k_quant_down_lds<6, UCOLS, MODE>), grid, dim3(64 * sq_waves<6>()), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_quant_down_lds<8, UCOLS, MODE>), grid, dim3(64 * sq_waves<8>()), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int quant_down_tiles(int r0, int rt) {
  (void)r0;
  return (rt + 31) / 32;  // the low-rank width in pairs of 16-wide tiles, padded
}

int quant_down_splits(int64_t M, int64_t K, int rt) {
  if (rt == 0) return 1;
  if (use_rows_kernel(M, rt)) {  // 128-row stripes; about one workgroup per CU
    const int64_t stripes = (M + QR_ROWS - 1) / QR_ROWS;
    const int64_t nchunks = (K + CHUNK - 1) / CHUNK;
    int64_t s = QD_TARGET_WGS / stripes;
    if (s > nchunks / 8) s = nchunks / 8;  // at least 8 chunks per range
    return (int)(s < 1 ? 1 : s);
  }
  const int64_t stripes = (M + QD_ROWS - 1) / QD_ROWS;
  const int64_t nchunks = (K + CHUNK - 1) / CHUNK;
  int64_t s = QD_TARGET_WGS / (stripes > 0 ? stripes : 1);  // about one workgroup per CU
  const int64_t maxs = nchunks / (2 * QD_WAVES);             // at least two chunks per wave
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

size_t quant_down_ut_bytes(int64_t M, int64_t K, int rt) {
  return use_rows_kernel(M, rt) ? (size_t)rt * K * 2 : 0;
}

size_t quant_down_partial_bytes(int64_t M, int64_t K, int r0, int rt) {
  (void)r0;
  const int S = quant_down_splits(M, K, rt);
  return S > 1 ? (size_t)S * M * rt * 4 : 0;
}

hipError_t launch_quant_down(const QuantDownArgs& a, bool x_bf16, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.rt % 16 != 0 || a.r0 % 16 != 0 || a.rt > 128 || a.r0 < 0 || a.r0 > a.rt) return hipErrorInvalidValue;
  const int tp = 2 * quant_down_tiles(a.r0, a.rt);  // 16-wide tiles, an even count
  const int S = quant_down_splits(a.M, a.K, a.rt);
  if (S > 1 && a.partials == nullptr) return hipErrorInvalidValue;
  hipError_t e;
  if (a.mode == QD_GELU_QUANT && (!x_bf16 || a.u_cols)) return hipErrorInvalidValue;
  if (a.mode == QD_DOWN && tp == 0) return hipErrorInvalidValue;
  const bool rows = x_bf16 && use_rows_kernel(a.M, a.rt) && (!a.u_cols || a.ut != nullptr);
  if (rows && a.u_cols) {
    // the backward's [B | L2] transposed once into the forward's layout, the only one the
    // row-split kernel reads (at 32760 x 15360, width 128, the kernel took 317 us on the
    // transposed operand against 425 us for a variant reading [B | L2] as stored, whose
    // transposed LDS reads issue twice the instructions); without the scratch the call
    // takes the staged kernel
    const int64_t blocks = a.K / 8 * (a.rt / 8);  // 8 x 8 blocks, one per thread
    hipLaunchKernelGGL(k_transpose_u, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream, a.d0, a.d1, a.r0,
                       a.rt - a.r0, a.K, a.ut);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    QuantDownArgs b = a;
    b.u_cols = false;
    b.d0 = a.ut;
    b.d1 = a.ut + (int64_t)a.r0 * a.K;
    e = a.mode == QD_DOWN ? launch_rows<QD_DOWN>(b, tp, S, stream) : launch_rows<QD_QUANT>(b, tp, S, stream);
  } else if (rows) {  // wide operand, many rows: the row-split kernel
    if (a.mode == QD_GELU_QUANT) e = launch_rows<QD_GELU_QUANT>(a, tp, S, stream);
    else if (a.mode == QD_DOWN) e = launch_rows<QD_DOWN>(a, tp, S, stream);
    else e = launch_rows<QD_QUANT>(a, tp, S, stream);
  } else if (x_bf16) {  // the staged kernel (whole-row loads, LDS-staged code stores)
    if (a.mode == QD_GELU_QUANT) e = launch_staged<false, QD_GELU_QUANT>(a, tp, S, stream);
    else if (a.mode == QD_DOWN) e = a.u_cols ? launch_staged<true, QD_DOWN>(a, tp, S, stream)
                                             : launch_staged<false, QD_DOWN>(a, tp, S, stream);
    else e = a.u_cols ? launch_staged<true, QD_QUANT>(a, tp, S, stream) : launch_staged<false, QD_QUANT>(a, tp, S, stream);
  } else if (a.mode == QD_DOWN) {  // fp32 input: the register kernel
    e = a.u_cols ? launch_reg<true, QD_DOWN>(a, tp, S, stream) : launch_reg<false, QD_DOWN>(a, tp, S, stream);
  } else {
    e = a.u_cols ? launch_reg<true, QD_QUANT>(a, tp, S, stream) : launch_reg<false, QD_QUANT>(a, tp, S, stream);
  }
  if (e != hipSuccess || S == 1) return e;
  const int64_t n4 = a.M * a.rt / 4;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a.partials, S, n4,
                     a.low);
  return hipGetLastError();
}

}  // namespace ft
