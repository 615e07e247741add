// Fused quantization + low-rank down-projection (FourTune §3.3 "LoRA Fusion": all
// three branches read the same input, so its quantization and every down-projection
// happen in one kernel and the input is read from HBM once).
//
//   forward : X -> Q(X), XL = bf16( bf16(X) [A; L1]^T )     D rows given (K-contiguous)
//   backward: G -> Q(G), GB = bf16( bf16(G) [B | L2] )       U rows given (rt-contiguous)
//
// HBM-bound: 2 (bf16) or 4 (fp32) bytes read and 0.5 written per input element, plus
// the small [M x rt] output. The down-projection runs on bf16 MFMA 16x16x32 straight
// from the registers the quantizer loaded.
//
// Work split. A workgroup of 4 waves owns 64 rows (two block rows) and one of S
// contiguous column ranges; wave w walks the range's 64-column chunks w, w+4, ....
// Register layout of a chunk = the 16x16x32 MFMA operand layout: lane l holds, for
// row group g (rows 16g + l%16) and column block b (32 columns), the 8 values at
// columns 32b + 8(l/16) .. +8. One load instruction thus reads 64 contiguous bytes
// of each of 16 rows (bf16); a 32x32 quantization block is row groups 2h, 2h+1 of
// column block b, its maximum met over the 64 lanes in VALU exchanges, and the E2M1
// conversion is the hardware one.
//
// Low-rank side, in 16-wide tiles (ranks are multiples of 16, so tiles never mix the
// two factors and need no padding): forward, tile t's rows of [A; L1] are loaded into
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
// depend on timing. (A last-arriving-workgroup reduction inside this kernel would
// need device-scope fences, which on this chip write back and invalidate the whole
// L2 of the issuing XCD: far dearer than a kernel boundary.)
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

template <typename T>
struct XChunk;

template <>
struct XChunk<bf16_t> {
  static constexpr int LOADS = 8;
  v4i v[4][2];  // [row group][column block]: 8 bf16
  __device__ void load(bufres r, const uint32_t (&row_off)[4], const bool (&row_ok)[4], int64_t c0, int64_t K,
                       int lq) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t c = c0 + 32 * b + 8 * lq;
        v[g][b] = buf_load16(r, sel_off(row_ok[g] && c < K, row_off[g] + (uint32_t)(c * 2)));
      }
  }
  __device__ uint32_t absmax(int g, int b) const {
    return umax(umax(bf16x2_absmax_bits(v[g][b].x), bf16x2_absmax_bits(v[g][b].y)),
                umax(bf16x2_absmax_bits(v[g][b].z), bf16x2_absmax_bits(v[g][b].w)));
  }
  __device__ uint32_t codes(int g, int b, float scale) const {
    return cvt8_bf16(v[g][b].x, v[g][b].y, v[g][b].z, v[g][b].w, scale);
  }
  __device__ v4i operand(int g, int b) const { return v[g][b]; }
};

// fp32 values are kept as float vectors: converting whole vectors (never single int
// lanes bit-cast to float) keeps the compiler's E2M1 conversion operands intact.
template <>
struct XChunk<float> {
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
    buf_load16_lds(first ? rd0 : rd1, sd + q * UStage<TP>::QSTRIDE, sel_off(nok, off));
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

template <typename T, int TP, bool UCOLS, int MODE>
__global__ __launch_bounds__(256) void k_quant_down(const QuantDownArgs a) {
  static_assert(TP % 2 == 0, "rank + stab_rank is a multiple of 32");
  constexpr int NS = (MODE == QD_QUANT || MODE == QD_GELU_QUANT) ? QD_STORES : 0;  // stores per chunk
  constexpr int RT = 16 * TP;
  constexpr int WAVE_LDS = UCOLS ? 2 * UStage<TP>::BYTES : 0;
  constexpr int RED = QD_WAVES * 4 * TP * 4 * 64 * 4;
  constexpr int SMEM = QD_WAVES * WAVE_LDS > RED ? QD_WAVES * WAVE_LDS : RED;
  constexpr int NX = XChunk<T>::LOADS, NU = UStage<TP>::LOADS;
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

  const bufres rx = make_buf(a.x, (uint64_t)a.M * a.ldx * sizeof(T));
  const bufres rcodes = make_buf(a.codes, (uint64_t)a.M * cpitch);
  const bufres rscales = make_buf(a.scales, (uint64_t)((a.M + 31) / 32) * nkb);
  uint32_t row_off[4];
  bool row_ok[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t row = r0 + 16 * g + lr;
    row_ok[g] = row < a.M;
    row_off[g] = (uint32_t)(row * a.ldx * sizeof(T));
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
  auto work = [&](const XChunk<T>& x, const DChunk<TP>& d, const lds_char* sd, int64_t ch) {
    const int64_t c0 = cstart(ch);
    if constexpr (MODE == QD_GELU_QUANT) {
      // x is the saved FC1 output P^ (bf16). H = GELU(P^) in fp32 for every element:
      // Q(H) is decided on these fp32 values, bf16(H) is the down-projection operand
      float hv[4][2][8];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t w[4] = {(uint32_t)x.v[g][b].x, (uint32_t)x.v[g][b].y, (uint32_t)x.v[g][b].z,
                                 (uint32_t)x.v[g][b].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hv[g][b][2 * e] = gelu_f(bf16_lo(w[e]));
            hv[g][b][2 * e + 1] = gelu_f(bf16_hi(w[e]));
          }
        }
      if constexpr (TP > 0) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          v4i xop[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            xop[g] = v4i{(int)pack_bf16x2(hv[g][b][0], hv[g][b][1]), (int)pack_bf16x2(hv[g][b][2], hv[g][b][3]),
                         (int)pack_bf16x2(hv[g][b][4], hv[g][b][5]), (int)pack_bf16x2(hv[g][b][6], hv[g][b][7])};
#pragma unroll
          for (int t = 0; t < TP; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[g][t] = mfma16(d.v[t][b], xop[g], acc[g][t]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t bc = c0 + 32 * b;
          const bool bok = bc < a.K;
          uint32_t m = 0;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = umax(m, __builtin_bit_cast(uint32_t, hv[2 * h + q][b][e]) & 0x7FFFFFFFu);
          const uint32_t sb = scale_byte_from_amax(wave_max_u32(m));
          const float scale = e8m0_to_f32_scale(sb);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int g = 2 * h + q;
            const int64_t row = r0 + 16 * g + lr;
            uint32_t cw = cvt8_f32(hv[g][b], scale);
            if (sb == 0xFFu) cw = 0;
            buf_store4(rcodes, sel_off(bok && row_ok[g], (uint32_t)(row * cpitch + ((bc + 8 * lq) >> 1))), cw);
          }
          buf_store1(rscales,
                     sel_off(bok && lane == 0 && r0 + 32 * h < a.M, (uint32_t)((r0 / 32 + h) * nkb + (bc >> 5))),
                     sb);
        }
      return;
    }
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

  // Two chunks per trip, each in its own register set (and LDS stage). The second may
  // lie past the range: it then loads zeros and stores nothing, which keeps the trip
  // branch-free and its memory-operation count fixed.
  XChunk<T> x0, x1;
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
    float* red = (float*)smem_raw;
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
    float* part = a.partials + ((int64_t)split * a.M) * RT;
    for (int e = tid; e < NI; e += 256) {
      const int l = e & 63, t = (e >> 6) % TP, g = e / (64 * TP);
      v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < QD_WAVES; ++w) {
        const float* src = red + ((((w * 4 + g) * TP + t) * 4) * 64 + l);
        s += v4f{src[0], src[64], src[128], src[192]};
      }
      const int64_t orow = r0 + 16 * g + (l & 15);
      const int col = 16 * t + 4 * (l >> 4);
      if (orow < a.M) {
        if (partial)
          *reinterpret_cast<v4f*>(part + orow * RT + col) = s;
        else
          *reinterpret_cast<uint2*>(a.low + orow * RT + col) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
      }
    }
  }
}

// Sum of the S column-range partials of each row, in range order, rounded once to
// bf16.
__global__ __launch_bounds__(256) void k_sum_partials(const float* __restrict__ partials, int S, int64_t n4,
                                                      bf16_t* __restrict__ low) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one v4f of [M x rt]
  if (i >= n4) return;
  const v4f* pv = reinterpret_cast<const v4f*>(partials);
  v4f s = pv[i];
  for (int sp = 1; sp < S; ++sp) s += pv[sp * n4 + i];
  *reinterpret_cast<uint2*>(low + 4 * i) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
}

template <typename T, bool UCOLS, int MODE>
hipError_t launch_t(const QuantDownArgs& a, int tp, int splits, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + QD_ROWS - 1) / QD_ROWS), (unsigned)splits), block(256);
  switch (tp) {
    case 0: hipLaunchKernelGGL((k_quant_down<T, 0, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_quant_down<T, 2, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_quant_down<T, 4, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((k_quant_down<T, 6, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_quant_down<T, 8, UCOLS, MODE>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int quant_down_tiles(int r0, int rt) { return (r0 + 31) / 32 + (rt - r0 + 31) / 32; }

int quant_down_splits(int64_t M, int64_t K, int rt) {
  if (rt == 0) return 1;
  const int64_t stripes = (M + QD_ROWS - 1) / QD_ROWS;
  const int64_t nchunks = (K + CHUNK - 1) / CHUNK;
  int64_t s = QD_TARGET_WGS / (stripes > 0 ? stripes : 1);  // about one workgroup per CU
  const int64_t maxs = nchunks / (2 * QD_WAVES);             // at least two chunks per wave
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

size_t quant_down_partial_bytes(int64_t M, int64_t K, int r0, int rt) {
  (void)r0;
  const int S = quant_down_splits(M, K, rt);
  return S > 1 ? (size_t)S * M * rt * 4 : 0;
}

hipError_t launch_quant_down(const QuantDownArgs& a, bool x_bf16, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.rt % 32 != 0 || a.r0 % 16 != 0 || a.rt > 128 || a.r0 < 0 || a.r0 > a.rt) return hipErrorInvalidValue;
  const int tp = a.rt / 16;
  const int S = quant_down_splits(a.M, a.K, a.rt);
  if (S > 1 && a.partials == nullptr) return hipErrorInvalidValue;
  hipError_t e;
  if (a.mode == QD_GELU_QUANT) {  // the saved P^: Q(GELU(P^)) and [A2; L1_2] down
    if (!x_bf16 || a.u_cols) return hipErrorInvalidValue;
    e = launch_t<bf16_t, false, QD_GELU_QUANT>(a, tp, S, stream);
  } else if (a.mode == QD_DOWN) {  // down-projection alone, either side
    if (tp == 0) return hipErrorInvalidValue;
    if (a.u_cols)
      e = x_bf16 ? launch_t<bf16_t, true, QD_DOWN>(a, tp, S, stream) : launch_t<float, true, QD_DOWN>(a, tp, S, stream);
    else
      e = x_bf16 ? launch_t<bf16_t, false, QD_DOWN>(a, tp, S, stream) : launch_t<float, false, QD_DOWN>(a, tp, S, stream);
  } else if (a.u_cols) {
    e = x_bf16 ? launch_t<bf16_t, true, QD_QUANT>(a, tp, S, stream) : launch_t<float, true, QD_QUANT>(a, tp, S, stream);
  } else {
    e = x_bf16 ? launch_t<bf16_t, false, QD_QUANT>(a, tp, S, stream) : launch_t<float, false, QD_QUANT>(a, tp, S, stream);
  }
  if (e != hipSuccess || S == 1) return e;
  const int64_t n4 = a.M * a.rt / 4;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a.partials, S, n4,
                     a.low);
  return hipGetLastError();
}

}  // namespace ft
