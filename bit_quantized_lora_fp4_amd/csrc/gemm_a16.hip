// 16-bit activation x 4-bit weight GEMM for the precision variants (FourTune §4,
// "Impact of Precision Configurations": W4A16G4, W4A4G16 and W4A16G16 keep the
// activations or the gradients in 16 bits while the weight stays 4-bit).
//
//   forward : out[M x N] = bf16(X)[M x K] deq Q(R)[N x K]^T + low[M x rt] U[N x rt]^T
//   backward: out[M x K] = bf16(G)[M x N] deq Q(R)[N x K]   + low[M x rt] D[rt x K]
//
// An E2M1 value times a power of two is exact in bf16, so the weight tile is
// dequantized to bf16 as it is staged in LDS (hardware v_cvt_scalef32_pk_bf16_fp4) and
// the product runs on bf16 MFMA 32x32x16 with fp32 accumulation. The low-rank
// up-projection continues the same reduction over rt more elements:
// [act | low] x [deq R | V]. Only the W4A4G4 configuration runs the 4-bit MFMA; this
// kernel is what the other configurations cost.
//
// Tiling: 128 x 128 output tile, reduction steps of 64, four waves of 64 x 64 (2 x 2
// MFMA tiles). Each step's operands go global -> registers -> LDS while the previous
// step's MFMAs run (two LDS buffers); the activation tile is staged [row][k], the
// weight tile [column][k] (forward) or [k][column] (backward, read transposed with
// ds_read_b64_tr_b16). The first MFMA operand is the weight side, so a lane's
// accumulator holds four consecutive output columns of one row; the result leaves
// through LDS as whole rows.
#include "common.h"
#include "gemm.h"

namespace ft {

namespace {

constexpr int QM = 128, QN = 128, QK = 64;
constexpr int QA_PITCH = QK * 2 + 16;        // activation row: 64 bf16 + 16 bytes
constexpr int QBF_PITCH = QK * 2 + 16;       // forward weight row (one output column)
constexpr int QBB_PITCH = QN * 2 + 32;       // backward weight row (one reduction index)
constexpr int QA_BYTES = QM * QA_PITCH;      // 18 KB
constexpr int QB_BYTES = (QN * QBF_PITCH > QK * QBB_PITCH) ? QN * QBF_PITCH : QK * QBB_PITCH;
constexpr int QSTAGE = QA_BYTES + QB_BYTES;  // one buffer
constexpr int QST_PITCH = 64 * 4 + 16;       // staged fp32 output row (64 columns)
constexpr int QST_WAVE = 64 * QST_PITCH;

__device__ __forceinline__ v16f mfma_bf16_q(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ void lds_st16(lds_char* p, v4i v) { *(__attribute__((address_space(3))) v4i*)p = v; }
__device__ __forceinline__ v4i lds_ld16(const lds_char* p) { return *(const __attribute__((address_space(3))) v4i*)p; }

// 32 FP4 codes (16 bytes, even element in the low nibble) times the block scale -> 32
// bf16 in four 16-byte words
__device__ __forceinline__ void deq32(v4i codes, uint32_t scale_byte, v4i (&out)[4]) {
  const float s = e8m0_to_f32_scale(scale_byte);
  const uint32_t w[4] = {(uint32_t)codes.x, (uint32_t)codes.y, (uint32_t)codes.z, (uint32_t)codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v4i o;
    o.x = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 0));
    o.y = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 1));
    o.z = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 2));
    o.w = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 3));
    if (scale_byte == 0xFFu) o = v4i{0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0};  // NaN block
    out[q] = o;
  }
}

template <typename T>
struct ActIO;
template <>
struct ActIO<bf16_t> {
  // 8 consecutive elements as 8 bf16
  static __device__ v4i load8(bufres r, uint32_t elem_off, bool ok) { return buf_load16(r, sel_off(ok, elem_off * 2)); }
};
template <>
struct ActIO<float> {
  static __device__ v4i load8(bufres r, uint32_t elem_off, bool ok) {
    const uint32_t o = sel_off(ok, elem_off * 4);
    const v4f a = __builtin_bit_cast(v4f, buf_load16(r, o));
    const v4f b = __builtin_bit_cast(v4f, buf_load16(r, o + 16));
    return v4i{(int)pack_bf16x2(a.x, a.y), (int)pack_bf16x2(a.z, a.w), (int)pack_bf16x2(b.x, b.y),
               (int)pack_bf16x2(b.z, b.w)};
  }
};

template <typename T, bool TRANS_B, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_gemm_a16(const GemmA16Args g) {
  __shared__ __align__(16) char lds_raw[2 * QSTAGE];
  lds_char* const lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t M = g.M, N = g.N, Kred = g.Kred;
  const int rt = g.rt, r0 = g.up_split;
  const int64_t m0 = (int64_t)blockIdx.y * QM, n0 = (int64_t)blockIdx.x * QN;
  const int KTQ = (int)((Kred + QK - 1) / QK);  // steps over the 4-bit weight
  const int KT = KTQ + (rt + QK - 1) / QK;       // then over the low-rank columns

  const bufres ract = make_buf(g.act, (uint64_t)M * g.ld_act * sizeof(T));
  const int64_t r_rows = TRANS_B ? Kred : N;      // rows of Q(R) (it is [N_lin x K_lin])
  const int64_t r_cols = TRANS_B ? N : Kred;
  const bufres rcode = make_buf(g.b_codes, (uint64_t)r_rows * (r_cols >> 1));
  const bufres rscl = make_buf(g.b_scales, (uint64_t)((r_rows + 31) >> 5) * (r_cols >> 5));
  const bufres rlow = make_buf(g.low, (uint64_t)M * rt * 2);
  const int s1 = rt - r0;
  const bufres rv0 = make_buf(g.up0, TRANS_B ? (uint64_t)r0 * N * 2 : (uint64_t)N * r0 * 2);
  const bufres rv1 = make_buf(g.up1, TRANS_B ? (uint64_t)s1 * N * 2 : (uint64_t)N * s1 * 2);

  // ---- staging registers of one step
  v4i ra[4];     // activation: 4 units of 8 elements
  v4i rb[4];     // weight: 4 units of 8 bf16 (low-rank steps) or 16 bytes of codes (rb[0])
  uint32_t rbs;  // scale byte of the codes

  // activation units: u = tid + 256 q (q < 4) -> row u / 8, k 8 (u % 8)
  auto load_step = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q, row = u >> 3, k = 8 * (u & 7);
      const int64_t m = m0 + row;
      if (kt < KTQ) {
        const int64_t kk = (int64_t)kt * QK + k;
        ra[q] = ActIO<T>::load8(ract, (uint32_t)(m * g.ld_act + kk), m < M && kk < Kred);
      } else {
        const int j = (kt - KTQ) * QK + k;
        ra[q] = buf_load16(rlow, sel_off(m < M && j < rt, (uint32_t)((m * rt + j) * 2)));
      }
    }
    if (kt < KTQ) {
      // one 32-element block row piece per thread
      if constexpr (!TRANS_B) {
        // weight tile [128 output columns n][64 k]: thread -> column tid/2, block half tid%2
        const int c = tid >> 1, h = tid & 1;
        const int64_t n = n0 + c, kb = (int64_t)kt * 2 + h;
        const bool ok = n < N && 32 * kb < Kred;
        rb[0] = buf_load16(rcode, sel_off(ok, (uint32_t)(n * (r_cols >> 1) + kb * 16)));
        rbs = buf_load1(rscl, sel_off(ok, (uint32_t)((n >> 5) * (r_cols >> 5) + kb)));
      } else {
        // weight tile [64 k (rows of R)][128 output columns]: thread -> row tid/4, 32 columns
        const int kr = tid >> 2, cu = tid & 3;
        const int64_t k = (int64_t)kt * QK + kr, c = n0 + 32 * cu;
        const bool ok = k < Kred && c < N;
        rb[0] = buf_load16(rcode, sel_off(ok, (uint32_t)(k * (r_cols >> 1) + (c >> 1))));
        rbs = buf_load1(rscl, sel_off(ok, (uint32_t)((k >> 5) * (r_cols >> 5) + (c >> 5))));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = tid + 256 * q;
        if constexpr (!TRANS_B) {
          // U tile [128 columns n][64 ranks]: unit -> column u/8, ranks 8 (u%8)
          const int c = u >> 3;
          const int j = (kt - KTQ) * QK + 8 * (u & 7);
          const int64_t n = n0 + c;
          const bool ok = n < N && j < rt;
          if (j < r0)  // uniform per 8-rank unit; r0 is a multiple of 16
            rb[q] = buf_load16(rv0, sel_off(ok, (uint32_t)((n * r0 + j) * 2)));
          else
            rb[q] = buf_load16(rv1, sel_off(ok, (uint32_t)((n * s1 + j - r0) * 2)));
        } else {
          // D tile [64 ranks][128 columns]: unit -> rank u/16, columns 8 (u%16)
          const int jr = u >> 4;
          const int j = (kt - KTQ) * QK + jr;
          const int64_t c = n0 + 8 * (u & 15);
          const bool ok = c < N && j < rt;
          if (j < r0)
            rb[q] = buf_load16(rv0, sel_off(ok, (uint32_t)(((int64_t)j * N + c) * 2)));
          else
            rb[q] = buf_load16(rv1, sel_off(ok, (uint32_t)(((int64_t)(j - r0) * N + c) * 2)));
        }
      }
    }
  };
  auto store_step = [&](int kt, lds_char* buf) __attribute__((always_inline)) {
    lds_char* sa = buf;
    lds_char* sb = buf + QA_BYTES;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q;
      lds_st16(sa + (u >> 3) * QA_PITCH + 16 * (u & 7), ra[q]);
    }
    if (kt < KTQ) {
      v4i d[4];
      deq32(rb[0], rbs, d);
      if constexpr (!TRANS_B) {
        const int c = tid >> 1, h = tid & 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) lds_st16(sb + c * QBF_PITCH + 64 * h + 16 * q, d[q]);
      } else {
        const int kr = tid >> 2, cu = tid & 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) lds_st16(sb + kr * QBB_PITCH + 64 * cu + 16 * q, d[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = tid + 256 * q;
        if constexpr (!TRANS_B)
          lds_st16(sb + (u >> 3) * QBF_PITCH + 16 * (u & 7), rb[q]);
        else
          lds_st16(sb + (u >> 4) * QBB_PITCH + 16 * (u & 15), rb[q]);
      }
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  load_step(0);
  store_step(0, lds);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    lds_char* cur = lds + (kt & 1) * QSTAGE;
    if (kt + 1 < KT) load_step(kt + 1);
    const lds_char* sa = cur;
    const lds_char* sb = cur + QA_BYTES;
#pragma unroll
    for (int s = 0; s < QK / 16; ++s) {
      v4i a[2], b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        a[j] = lds_ld16(sa + (wm * 64 + 32 * j + (lane & 31)) * QA_PITCH + 2 * (16 * s + 8 * (lane >> 5)));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (!TRANS_B)
          b[i] = lds_ld16(sb + (wn * 64 + 32 * i + (lane & 31)) * QBF_PITCH + 2 * (16 * s + 8 * (lane >> 5)));
        else
          b[i] = lds_tr16_pair(sb, QBB_PITCH, 16 * s, wn * 64 + 32 * i, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16_q(b[i], a[j], acc[i][j]);
    }
    if (kt + 1 < KT) store_step(kt + 1, lds + ((kt + 1) & 1) * QSTAGE);
    __syncthreads();
  }

  // acc[i][j][r] = out[row m0 + 64 wm + 32 j + lane%32][col n0 + 64 wn + 32 i + 8(r/4) + 4(lane/32) + r%4]
  lds_char* stw = lds + wave * QST_WAVE;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v16f& t = acc[i][j];
        const v4f w = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
        *(__attribute__((address_space(3))) v4f*)(stw + (32 * j + (lane & 31)) * QST_PITCH +
                                                  4 * (32 * i + 8 * q + 4 * (lane >> 5))) = w;
      }
  __syncthreads();
  const bufres rout = make_buf(g.out, (uint64_t)M * g.ldo * (OUT_BF16 ? 2 : 4));
#pragma unroll
  for (int it = 0; it < 8; ++it) {  // 8 rows x 8 columns per lane... 64 rows, 8 lanes per row
    const int rl = 8 * it + (lane >> 3), cl = 8 * (lane & 7);
    const lds_char* p = stw + rl * QST_PITCH + 4 * cl;
    const v4f x0 = *(const __attribute__((address_space(3))) v4f*)p;
    const v4f x1 = *(const __attribute__((address_space(3))) v4f*)(p + 16);
    const int64_t row = m0 + wm * 64 + rl, col = n0 + wn * 64 + cl;
    if (row < M && col < N) {
      if constexpr (OUT_BF16) {
        const v4i o = {(int)pack_bf16x2(x0[0], x0[1]), (int)pack_bf16x2(x0[2], x0[3]), (int)pack_bf16x2(x1[0], x1[1]),
                       (int)pack_bf16x2(x1[2], x1[3])};
        __builtin_amdgcn_raw_buffer_store_b128(o, rout, (int)((row * g.ldo + col) * 2), 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, x0), rout, (int)((row * g.ldo + col) * 4), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, x1), rout, (int)((row * g.ldo + col) * 4 + 16),
                                               0, 0);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_a16(const GemmA16Args& g, bool act_bf16, bool trans_b, bool out_bf16, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.rt < 0 || g.rt % 16 != 0 || g.rt > 128 || g.up_split % 16 != 0 || g.up_split > g.rt || g.N % 32 != 0 ||
      g.Kred % 32 != 0 || g.ld_act % 8 != 0 || g.ldo % 8 != 0)
    return hipErrorInvalidValue;
  const uint64_t act_bytes = (uint64_t)g.M * g.ld_act * (act_bf16 ? 2 : 4);
  const uint64_t out_bytes = (uint64_t)g.M * g.ldo * (out_bf16 ? 2 : 4);
  if (act_bytes >= 0xFFFFFF00ull || out_bytes >= 0xFFFFFF00ull) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((g.N + QN - 1) / QN), (unsigned)((g.M + QM - 1) / QM));
  if (grid.y > 65535u) return hipErrorInvalidValue;
#define FT_A16_LAUNCH(T, TB, OB) hipLaunchKernelGGL((k_gemm_a16<T, TB, OB>), grid, dim3(256), 0, stream, g)
  if (act_bf16) {
    if (trans_b) { if (out_bf16) FT_A16_LAUNCH(bf16_t, true, true); else FT_A16_LAUNCH(bf16_t, true, false); }
    else { if (out_bf16) FT_A16_LAUNCH(bf16_t, false, true); else FT_A16_LAUNCH(bf16_t, false, false); }
  } else {
    if (trans_b) { if (out_bf16) FT_A16_LAUNCH(float, true, true); else FT_A16_LAUNCH(float, true, false); }
    else { if (out_bf16) FT_A16_LAUNCH(float, false, true); else FT_A16_LAUNCH(float, false, false); }
  }
#undef FT_A16_LAUNCH
  return hipGetLastError();
}

}  // namespace ft
