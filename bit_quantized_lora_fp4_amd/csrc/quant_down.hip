// Fused quantization + low-rank down-projection (FourTune §3.3 "LoRA Fusion": all
// three branches read the same input, so its quantization and every down-projection
// happen in one kernel and the input is read from HBM once).
//
//   forward : X -> Q(X), XL = bf16( bf16(X) [A; L1]^T )     D rows given (K-contiguous)
//   backward: G -> Q(G), GB = bf16( bf16(G) [B | L2] )       U rows given (rt-contiguous)
//
// HBM-bound: 2 (bf16) or 4 (fp32) bytes read and 0.5 written per input element, plus
// the small [M x rt] output. The down-projection runs on bf16 MFMA (32x32x16) straight
// from the registers the quantizer loaded.
//
// Work split. A workgroup of 4 waves owns 64 rows (two block rows) and one of S
// contiguous column ranges; wave w walks the range's 64-column chunks w, w+4, ....
// Inside a chunk, lane l holds row l%32 of each 32-row half and, for each of the 4
// 16-column steps, columns (l/32)*8 .. +8 of the step: the bf16 MFMA operand layout;
// for the quantizer each 32x32 block is two steps. Block maxima meet over the 64 lanes
// in VALU exchanges; the E2M1 conversion is the hardware one.
//
// Pipeline. Each wave alternates two register sets for its input chunks and two LDS
// stages for the low-rank operand of those chunks, which it fetches itself with
// direct-to-LDS buffer loads: chunk i+1's input and chunk i+2's operand are in flight
// while chunk i is worked on. Every load and store is issued unconditionally (masked
// lanes use out-of-range offsets), so the number of memory operations between two
// points is fixed and the operand stages are awaited with exact vmcnt counts.
//
// The low-rank side is laid out in padded 32-row tiles: the first ceil(r0/32) tiles
// hold the first factor ([A] or [B]'s columns), the rest the second, so every tile has
// a single source and no per-lane choice of buffer is needed.
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
constexpr int QD_ROWS = 64;   // rows per workgroup (two block rows)
constexpr int CHUNK = 64;     // columns per wave iteration (two blocks)
constexpr int QD_STORES = 12;  // stores per chunk: 8 code words + 4 scale bytes

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T>
struct XChunk;

template <>
struct XChunk<bf16_t> {
  static constexpr int LOADS = 8;
  v4i v[2][4];  // [row half][step]: 8 bf16 at columns c0 + 16s + 8*(l/32)
  __device__ void load(bufres r, const uint32_t row_off[2], const bool row_ok[2], int64_t c0, int64_t K,
                       int half) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t c = c0 + 16 * s + 8 * half;
        v[h][s] = buf_load16(r, sel_off(row_ok[h] && c < K, row_off[h] + (uint32_t)(c * 2)));
      }
  }
  __device__ uint32_t absmax(int h, int s) const {
    return umax(umax(bf16x2_absmax_bits(v[h][s].x), bf16x2_absmax_bits(v[h][s].y)),
                umax(bf16x2_absmax_bits(v[h][s].z), bf16x2_absmax_bits(v[h][s].w)));
  }
  __device__ uint32_t codes(int h, int s, float scale) const {
    return cvt8_bf16(v[h][s].x, v[h][s].y, v[h][s].z, v[h][s].w, scale);
  }
  __device__ v4i operand(int h, int s) const { return v[h][s]; }
};

// fp32 values are kept as float vectors: converting whole vectors (never single int
// lanes bit-cast to float) keeps the compiler's E2M1 conversion operands intact.
template <>
struct XChunk<float> {
  static constexpr int LOADS = 16;
  v4f v[2][4][2];
  __device__ void load(bufres r, const uint32_t row_off[2], const bool row_ok[2], int64_t c0, int64_t K,
                       int half) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t c = c0 + 16 * s + 8 * half;
        const uint32_t off = sel_off(row_ok[h] && c < K, row_off[h] + (uint32_t)(c * 4));
        v[h][s][0] = __builtin_bit_cast(v4f, buf_load16(r, off));
        v[h][s][1] = __builtin_bit_cast(v4f, buf_load16(r, off + 16));  // OOB + 16 is still OOB
      }
  }
  __device__ uint32_t absmax(int h, int s) const {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const v4i w = __builtin_bit_cast(v4i, v[h][s][q]) & 0x7FFFFFFF;
      m = umax(m, umax(umax((uint32_t)w.x, (uint32_t)w.y), umax((uint32_t)w.z, (uint32_t)w.w)));
    }
    return m;
  }
  __device__ uint32_t codes(int h, int s, float scale) const {
    const v4f a = v[h][s][0], b = v[h][s][1];
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return cvt8_f32(f, scale);
  }
  __device__ v4i operand(int h, int s) const {  // bf16(x), round to nearest even
    const v4f a = v[h][s][0], b = v[h][s][1];
    return v4i{(int)pack_bf16x2(a.x, a.y), (int)pack_bf16x2(a.z, a.w), (int)pack_bf16x2(b.x, b.y),
               (int)pack_bf16x2(b.z, b.w)};
  }
};

// One LDS stage of a chunk's low-rank operand (TP padded 32-row tiles).
//   forward : block (t, s) = D tile t, columns c0 + 16s .. +16, as the MFMA's first
//             operand: lane l's 16 bytes (row 32t + l%32, 8 columns at 8*(l/32)) at
//             ((t*4 + s)*64 + l)*16.
//   backward: block q = 16-byte unit q (padded columns 8q .. 8q+8) of the chunk's 64
//             rows of [B | L2], row n - c0 at 16*(n - c0); blocks are QSTRIDE apart
//             (64 bytes of padding keep the transposed reads free of bank conflicts).
template <int TP, bool UCOLS>
struct DStage {
  static constexpr int ND = 4 * TP;  // 16-byte direct-to-LDS loads per lane per chunk
  static constexpr int QSTRIDE = UCOLS ? 1024 + 64 : 1024;
  static constexpr int BYTES = ND * QSTRIDE;
};

template <int TP, bool UCOLS>
__device__ __forceinline__ void fetch_d(lds_char* sd, bufres rd0, bufres rd1, int ta, int r0, int rt,
                                        int64_t c0, int64_t K, int lane) {
  using DS = DStage<TP, UCOLS>;
  if constexpr (!UCOLS) {
    const int half = lane >> 5;
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const bool first = t < ta;  // uniform
      const int j = (first ? 32 * t : 32 * (t - ta)) + (lane & 31);
      const bool jok = first ? j < r0 : j < rt - r0;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t c = c0 + 16 * s + 8 * half;
        const uint32_t off = sel_off(jok && c < K, (uint32_t)(((int64_t)j * K + c) * 2));
        buf_load16_lds(first ? rd0 : rd1, sd + (t * 4 + s) * DS::QSTRIDE, off);
      }
    }
  } else {
    const int64_t n = c0 + lane;
    const bool nok = n < K;
#pragma unroll
    for (int q = 0; q < 4 * TP; ++q) {
      const bool first = q < 4 * ta;  // uniform
      const int j0 = first ? 8 * q : 8 * (q - 4 * ta);
      const bool ok = nok && (first ? j0 < r0 : j0 < rt - r0);
      const uint32_t off = first ? (uint32_t)((n * r0 + j0) * 2) : (uint32_t)((n * (rt - r0) + j0) * 2);
      buf_load16_lds(first ? rd0 : rd1, sd + q * DS::QSTRIDE, sel_off(ok, off));
    }
  }
}

// Backward operand from the [q][n] stage: for each padded tile t, lane l receives
// column 32t + l%32 of rows n0 + 8*(l/32) .. +8, via two ds_read_b64_tr_b16 per tile
// (see lds_tr16_pair for the instruction's lane pattern). The reads are issued from
// inline asm, which waits for them itself: the compiler would otherwise hold each LDS
// read back until every direct-to-LDS load in flight (including the next chunk's
// operand) had landed.
template <int QSTRIDE>
__device__ __forceinline__ uint32_t tr16_qn_addr(const lds_char* base, int n0, int j0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int j = j0 + 16 * (g & 1) + 4 * (s & 3);
  const int n = n0 + 8 * (g >> 1) + (s >> 2);
  return (uint32_t)(uintptr_t)(base + (j >> 3) * QSTRIDE + n * 16 + (j & 7) * 2);
}

template <int TP, int QSTRIDE>
__device__ __forceinline__ void lds_tr16_qn_tiles(const lds_char* base, int n0, int lane, v4i* out) {
#pragma unroll
  for (int t = 0; t < TP; t += 2) {
    const uint32_t p0 = tr16_qn_addr<QSTRIDE>(base, n0, 32 * t, lane);
    if (t + 1 < TP) {
      const uint32_t p1 = tr16_qn_addr<QSTRIDE>(base, n0, 32 * (t + 1), lane);
      v2i a, b, c, d;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %4 offset:64\n\t"
          "ds_read_b64_tr_b16 %2, %5\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
          : "v"(p0), "v"(p1)
          : "memory");
      out[t] = v4i{a.x, a.y, b.x, b.y};
      out[t + 1] = v4i{c.x, c.y, d.x, d.y};
    } else {
      v2i a, b;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %2\n\t"
          "ds_read_b64_tr_b16 %1, %2 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a), "=&v"(b)
          : "v"(p0)
          : "memory");
      out[t] = v4i{a.x, a.y, b.x, b.y};
    }
  }
}

template <typename T, int TP, bool UCOLS, int MODE>
__global__ __launch_bounds__(256) void k_quant_down(const QuantDownArgs a) {
  using DS = DStage<TP, UCOLS>;
  constexpr int NS = MODE == QD_QUANT ? QD_STORES : 0;  // stores per chunk
  constexpr int RTP = 32 * TP;  // padded low-rank width
  constexpr int WAVE_LDS = 2 * DS::BYTES;
  constexpr int RED = QD_WAVES * 2 * TP * 16 * 64 * 4;
  constexpr int SMEM = QD_WAVES * WAVE_LDS > RED ? QD_WAVES * WAVE_LDS : RED;
  constexpr int NX = XChunk<T>::LOADS, ND = DS::ND;
  __shared__ __align__(16) char smem_raw[SMEM > 0 ? SMEM : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * QD_ROWS;
  const int split = blockIdx.y, S = gridDim.y;
  const int64_t nchunks = (a.K + CHUNK - 1) / CHUNK;
  const int64_t per = (nchunks + S - 1) / S;
  const int64_t ch0 = split * per, ch1 = min(nchunks, ch0 + per);
  const int64_t cpitch = a.K >> 1, nkb = a.K >> 5;
  const int ta = (a.r0 + 31) / 32;  // padded tiles of the first factor

  const bufres rx = make_buf(a.x, (uint64_t)a.M * a.ldx * sizeof(T));
  const bufres rcodes = make_buf(a.codes, (uint64_t)a.M * cpitch);
  const bufres rscales = make_buf(a.scales, (uint64_t)((a.M + 31) / 32) * nkb);
  uint32_t row_off[2];
  bool row_ok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t row = r0 + 32 * h + (lane & 31);
    row_ok[h] = row < a.M;
    row_off[h] = (uint32_t)(row * a.ldx * sizeof(T));
  }
  const bufres rd0 = make_buf(a.d0, (uint64_t)a.K * a.r0 * 2);
  const bufres rd1 = make_buf(a.d1, (uint64_t)a.K * (a.rt - a.r0) * 2);

  v16f acc[2][TP > 0 ? TP : 1];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[h][t] = v16f{};

  lds_char* sd0 = (lds_char*)smem_raw + wave * WAVE_LDS;
  lds_char* sd1 = sd0 + DS::BYTES;
  // chunks past the range move nothing: their column start is K, so every access is OOB
  auto cstart = [&](int64_t ch) { return ch < ch1 ? ch * CHUNK : a.K; };
  auto fetch = [&](lds_char* sd, int64_t ch) {
    if constexpr (TP > 0) fetch_d<TP, UCOLS>(sd, rd0, rd1, ta, a.r0, a.rt, cstart(ch), a.K, lane);
  };

  auto work = [&](const XChunk<T>& x, const lds_char* sd, int64_t ch) {
    const int64_t c0 = cstart(ch);
    // ---- down-projection: first MFMA operand the low-rank side (rows j), second the
    // input (rows m): a lane's accumulators hold 4 consecutive j of one row m
    if constexpr (TP > 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4i xop[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          xop[h] = x.operand(h, s);
          if constexpr (MODE == QD_GELU_DOWN)  // bf16(GELU(P^)), P^ the saved FC1 output
            xop[h] = v4i{(int)gelu_bf16x2((uint32_t)xop[h].x), (int)gelu_bf16x2((uint32_t)xop[h].y),
                         (int)gelu_bf16x2((uint32_t)xop[h].z), (int)gelu_bf16x2((uint32_t)xop[h].w)};
        }
        v4i dtr[TP];
        if constexpr (UCOLS) lds_tr16_qn_tiles<TP, DS::QSTRIDE>(sd, 16 * s, lane, dtr);
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          v4i dv;
          if constexpr (UCOLS) dv = dtr[t];
          else dv = *(const __attribute__((address_space(3))) v4i*)(sd + ((t * 4 + s) * 64 + lane) * 16);
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[h][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dv),
                                                                __builtin_bit_cast(bf16x8, xop[h]),
                                                                acc[h][t], 0, 0, 0);
        }
      }
    }
    // ---- quantize the chunk's four 32x32 blocks (2 row halves x 2 column blocks)
    if constexpr (MODE == QD_QUANT)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t bc = c0 + 32 * b;
        const bool bok = bc < a.K;
        const uint32_t amax = wave_max_u32(umax(x.absmax(h, 2 * b), x.absmax(h, 2 * b + 1)));
        const uint32_t sb = scale_byte_from_amax(amax);
        const float scale = e8m0_to_f32_scale(sb);
        const int64_t row = r0 + 32 * h + (lane & 31);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t cw = x.codes(h, 2 * b + q, scale);
          if (sb == 0xFFu) cw = 0;
          buf_store4(rcodes, sel_off(bok && row_ok[h], (uint32_t)(row * cpitch + ((bc + 16 * q + 8 * half) >> 1))),
                     cw);
        }
        buf_store1(rscales,
                   sel_off(bok && lane == 0 && r0 + 32 * h < a.M, (uint32_t)((r0 / 32 + h) * nkb + (bc >> 5))), sb);
      }
  };

  // Two chunks per trip, each in its own register set and operand stage. The second
  // may lie past the range: it then loads zeros and stores nothing, which keeps the
  // trip branch-free and its memory-operation count fixed.
  // The empty asm statements with a memory clobber pin the order of the groups of
  // memory operations, which the vmcnt counts below rely on.
  XChunk<T> x0, x1;
  int64_t ch = ch0 + wave;
  fetch(sd0, ch);
  asm volatile("" ::: "memory");
  x0.load(rx, row_off, row_ok, cstart(ch), a.K, half);
  asm volatile("" ::: "memory");
  // Out-of-range stores standing in for a chunk's stores: the loop is entered with the
  // same sequence of outstanding memory operations as each later trip, so the
  // compiler's waits for x0 at the top of the loop are no stricter than needed.
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    uint32_t off = BUF_OOB + 16u * i;  // distinct, opaque: none may be merged away
    asm volatile("" : "+v"(off));
    buf_store4(rcodes, off, 0u);
  }
  asm volatile("" ::: "memory");
  fetch(sd1, ch + QD_WAVES);
  if constexpr (TP > 0) wait_vmcnt<NX + NS + ND>();  // operand of chunk ch in sd0
  __builtin_amdgcn_sched_barrier(0);
  // (scheduling barriers keep each half's arithmetic after the wait that guards it)
  for (; ch < ch1; ch += 2 * QD_WAVES) {
    x1.load(rx, row_off, row_ok, cstart(ch + QD_WAVES), a.K, half);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    work(x0, sd0, ch);
    if constexpr (TP > 0) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // sd0 reads done before it is refilled
      fetch(sd0, ch + 2 * QD_WAVES);
      wait_vmcnt<NX + NS + ND>();  // operand of chunk ch + 4 in sd1
    }
    __builtin_amdgcn_sched_barrier(0);
    x0.load(rx, row_off, row_ok, cstart(ch + 2 * QD_WAVES), a.K, half);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    work(x1, sd1, ch + QD_WAVES);
    if constexpr (TP > 0) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fetch(sd1, ch + 3 * QD_WAVES);
      wait_vmcnt<NX + NS + ND>();  // operand of chunk ch + 8 in sd0
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (TP > 0) {
    // ---- sum the 4 waves' partials (LDS), then this range's [64 x rt] result. The
    // stages alias the reduction area: let every direct-to-LDS load land first.
    wait_vmcnt<0>();
    __syncthreads();
    float* red = (float*)smem_raw;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < TP; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(((wave * 2 + h) * TP + t) * 16 + r) * 64 + lane] = acc[h][t][r];
    __syncthreads();
    // padded column -> column of the output (or -1 for padding)
    auto real_col = [&](int pc) {
      const int t = pc >> 5;
      if (t < ta) return pc < a.r0 ? pc : -1;
      const int j = pc - 32 * ta;
      return j < a.rt - a.r0 ? a.r0 + j : -1;
    };
    // item e of the range result: (h, t, rq, l) -> row 32h + l%32, the 4 padded columns
    // 32t + 8rq + 4(l/32) .. +4 (accumulator registers 4rq .. 4rq+3)
    constexpr int NI = 2 * TP * 4 * 64;
    const bool partial = S > 1;
    float* part = a.partials + ((int64_t)split * a.M) * RTP;
    for (int e = tid; e < NI; e += 256) {
      const int l = e & 63, rq = (e >> 6) & 3, t = (e >> 8) % TP, h = e / (TP * 256);
      v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < QD_WAVES; ++w) {
        const float* src = red + ((((w * 2 + h) * TP + t) * 16 + 4 * rq) * 64 + l);
        s += v4f{src[0], src[64], src[128], src[192]};
      }
      const int64_t orow = r0 + 32 * h + (l & 31);
      const int pcol = 32 * t + 8 * rq + 4 * (l >> 5);
      if (orow < a.M) {
        if (partial) {
          *reinterpret_cast<v4f*>(part + orow * RTP + pcol) = s;
        } else {
          const int oc = real_col(pcol);  // the 4 columns share one source (multiples of 16)
          if (oc >= 0)
            *reinterpret_cast<uint2*>(a.low + orow * a.rt + oc) =
                make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
        }
      }
    }
  }
}

// Sum of the S column-range partials of each row, in range order, rounded once to
// bf16 and written to the row's real (unpadded) columns.
__global__ __launch_bounds__(256) void k_sum_partials(const float* __restrict__ partials, int S, int64_t M,
                                                      int rtp, int r0, int rt, bf16_t* __restrict__ low) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one v4f of [M x rtp]
  if (i >= M * rtp / 4) return;
  const int64_t row = (4 * i) / rtp;
  const int pc = (int)((4 * i) % rtp);
  const int ta = (r0 + 31) / 32, t = pc >> 5;
  int oc;
  if (t < ta) oc = pc < r0 ? pc : -1;
  else oc = (pc - 32 * ta) < rt - r0 ? r0 + (pc - 32 * ta) : -1;
  if (oc < 0) return;
  const v4f* pv = reinterpret_cast<const v4f*>(partials);
  const int64_t stride = M * rtp / 4;
  v4f s = pv[i];
  for (int sp = 1; sp < S; ++sp) s += pv[sp * stride + i];
  *reinterpret_cast<uint2*>(low + row * rt + oc) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
}

template <typename T, bool UCOLS, int MODE>
hipError_t launch_t(const QuantDownArgs& a, int tp, int splits, hipStream_t stream) {
  dim3 grid((unsigned)((a.M + QD_ROWS - 1) / QD_ROWS), (unsigned)splits), block(256);
  switch (tp) {
    case 0: hipLaunchKernelGGL((k_quant_down<T, 0, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((k_quant_down<T, 1, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_quant_down<T, 2, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((k_quant_down<T, 3, UCOLS, MODE>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_quant_down<T, 4, UCOLS, MODE>), grid, block, 0, stream, a); break;
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
  int64_t s = 448 / (stripes > 0 ? stripes : 1);
  const int64_t maxs = nchunks / (2 * QD_WAVES);  // at least two chunks per wave
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

size_t quant_down_partial_bytes(int64_t M, int64_t K, int r0, int rt) {
  const int S = quant_down_splits(M, K, rt);
  return S > 1 ? (size_t)S * M * 32 * quant_down_tiles(r0, rt) * 4 : 0;
}

hipError_t launch_quant_down(const QuantDownArgs& a, bool x_bf16, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int tp = quant_down_tiles(a.r0, a.rt);
  if (tp > QD_MAX_TILES) return hipErrorInvalidValue;
  const int S = quant_down_splits(a.M, a.K, a.rt);
  if (S > 1 && a.partials == nullptr) return hipErrorInvalidValue;
  hipError_t e;
  if (a.mode == QD_GELU_DOWN) {  // the saved FC1 output P^: bf16, [A2; L1_2] rows
    if (!x_bf16 || a.u_cols || tp == 0) return hipErrorInvalidValue;
    e = launch_t<bf16_t, false, QD_GELU_DOWN>(a, tp, S, stream);
  } else if (a.mode == QD_DOWN) {  // dP^ (bf16) against [B1 | L2_1]
    if (!x_bf16 || !a.u_cols || tp == 0) return hipErrorInvalidValue;
    e = launch_t<bf16_t, true, QD_DOWN>(a, tp, S, stream);
  } else if (a.u_cols) {
    e = x_bf16 ? launch_t<bf16_t, true, QD_QUANT>(a, tp, S, stream) : launch_t<float, true, QD_QUANT>(a, tp, S, stream);
  } else {
    e = x_bf16 ? launch_t<bf16_t, false, QD_QUANT>(a, tp, S, stream) : launch_t<float, false, QD_QUANT>(a, tp, S, stream);
  }
  if (e != hipSuccess || S == 1) return e;
  const int64_t items = a.M * 32 * tp / 4;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a.partials, S,
                     a.M, 32 * tp, a.r0, a.rt, a.low);
  return hipGetLastError();
}

}  // namespace ft
