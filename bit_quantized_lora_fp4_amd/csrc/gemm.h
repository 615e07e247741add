// Argument blocks and launchers of the GEMM-shaped kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace ft {

// 4-bit backbone GEMM with the low-rank up-projection accumulated in its epilogue.
//   forward : out[M x N] = deq A[M x Kred] * deq R[N x Kred]^T + low[M x rt] * U[N x rt]^T
//             U row q = up0[q*up0_ld + 0 .. up_split) ++ up1[q*up1_ld + 0 .. rt-up_split)
//             ([B | L2]: up0 = B, up1 = L2)
//   backward: out[M x N] = deq A[M x Kred] * deq R[Kred x N]   + low[M x rt] * D[rt x N]
//             D row j = up0 row j (j < up_split) or up1 row j - up_split, row strides
//             up0_ld / up1_ld ([A; L1]: up0 = A, up1 = L1)
// A and R are MXFP4 (codes + 32x32-block E8M0 scales).
// The LoRA gradients' row-range sum: dA [r x K] and dB [N x r] from the S fp32 partials
// k_lora_grad leaves (one [rp x q] tile per q output columns, dA tiles first; range sp
// of tile t at (sp * ntiles + t) * rp * q floats). Run by k_lora_reduce, or by extra
// workgroups appended to the backward GEMM's launch (which needs none of it and leaves
// CUs idle when its tile count is not a multiple of 256).
struct LoraReduce {
  const float* partials;
  float* dA;
  float* dB;
  int64_t K, N;
  int r, S, rp, q, ntiles;
  int64_t items;  // v4f outputs (tile elements / 4 over all tiles); 0: no reduction
};

// Output v4f i of the sum: the partials of all S ranges in range order.
__device__ __forceinline__ void lora_reduce_item(const LoraReduce& t, int64_t i) {
  const int ne4 = t.rp * t.q / 4;
  const int tile = (int)(i / ne4), idx = 4 * (int)(i % ne4);
  const int tilesA = (int)((t.K + t.q - 1) / t.q);
  const bool jobA = tile < tilesA;
  const int64_t q0 = (int64_t)(jobA ? tile : tile - tilesA) * t.q;
  const int64_t nbig = jobA ? t.K : t.N;
  int p, q;
  if (jobA) { p = idx / t.q; q = idx % t.q; }
  else { q = idx / t.rp; p = idx % t.rp; }
  if (p >= t.r || q0 + q >= nbig) return;
  const v4f s = sum_ranges(reinterpret_cast<const v4f*>(t.partials) + i, t.S, (int64_t)t.ntiles * ne4);
  if (jobA) *reinterpret_cast<v4f*>(t.dA + (int64_t)p * t.K + q0 + q) = s;
  else *reinterpret_cast<v4f*>(t.dB + (q0 + q) * t.r + p) = s;
}

struct GemmArgs {
  const uint8_t* a_codes;   // [M x Kred/2]
  const uint8_t* a_scales;  // [ceil(M/32) x Kred/32]
  const uint8_t* b_codes;   // Q(R) codes, b_pitch bytes per row
  const uint8_t* b_scales;  // Q(R) scales, row-major over R's blocks
  int64_t b_pitch;
  int64_t M, N, Kred;
  const bf16_t* low;        // [M x rt]
  int rt;
  const bf16_t* up0;
  int64_t up0_ld;
  const bf16_t* up1;
  int64_t up1_ld;
  int up_split;
  void* out;                // [M x N] fp32 or bf16, row stride ldo
  int64_t ldo;
  // MLP backward epilogue (transposed GEMM, bf16 output; FourTune §3.3 "MLP Fusion"):
  //   GEMM_EPI_DGELU_Q: dP = result * GELU'(pre); out = bf16(dP); Q(dP) -> q_codes/q_scales
  //                     (pre = the saved P^ [M x N] bf16, row stride N)
  // (The forward's GELU + Q(H) runs in the quantize + down-projection pass over P^,
  // QD_GELU_QUANT.)
  int epi;
  const bf16_t* pre;
  uint8_t* q_codes;         // [M x N/2]
  uint8_t* q_scales;        // [ceil(M/32) x N/32]
  float* dbg;               // optional: the fp32 dP that Q(dP) quantized, [M x N]
  // optional work for workgroups past the output tiles (backward only; items = 0: none)
  LoraReduce tail;
};

enum { GEMM_EPI_NONE = 0, GEMM_EPI_DGELU_Q = 2 };

hipError_t launch_gemm_mx4(const GemmArgs& g, bool trans_b, bool out_bf16, hipStream_t stream);
// Longest reduction the GEMM supports (its block scales are staged in LDS once).
constexpr int64_t GEMM_MAX_KRED = 16384;

// Fused quantize + down-projection over the rows of x [M x K] (row stride ldx):
// Q(x) -> codes/scales, low[M x rt] = bf16( bf16(x) * D^T ).
//   u_cols = false: D row j = d0 row j (j < r0) or d1 row j - r0, each K-contiguous
//                   with row stride K ([A; L1] in the forward).
//   u_cols = true : D^T row n = d0[n*r0 .. +r0] ++ d1[n*(rt-r0) .. +(rt-r0)]
//                   ([B | L2] in the backward, read as stored).
// The K range is split S = quant_down_splits(M, K, rt) ways; with S > 1 the launch
// needs quant_down_partial_bytes(M, K, r0, rt) bytes of fp32 partials, which a second
// kernel sums in a fixed order.
// mode: QD_QUANT (as above); QD_DOWN: no quantization; QD_GELU_QUANT: x = the saved
// FC1 output P^ (bf16), H = GELU(P^) in fp32 -> Q(H), low = bf16(bf16(H) D^T); when
// hdbg is not NULL the fp32 H that Q(H) quantized is also stored there ([M x K]).
enum { QD_QUANT = 0, QD_DOWN = 2, QD_GELU_QUANT = 3 };
struct QuantDownArgs {
  int mode;
  const void* x;
  int64_t M, K, ldx;
  uint8_t* codes;
  uint8_t* scales;
  const bf16_t* d0;
  const bf16_t* d1;
  int r0;
  int rt;
  bool u_cols;
  bf16_t* low;
  float* partials;
  float* hdbg;  // QD_GELU_QUANT only, optional
  // u_cols only, optional: scratch of quant_down_ut_bytes(M, K, rt) bytes. Where the
  // wide-operand kernel runs, [B | L2] is first transposed into it ([rt x K], the
  // forward's layout), which that kernel reads with fewer LDS instructions.
  bf16_t* ut;
};

hipError_t launch_quant_down(const QuantDownArgs& a, bool x_bf16, hipStream_t stream);
// Bytes of the optional u_cols scratch (0 where it would not be used).
size_t quant_down_ut_bytes(int64_t M, int64_t K, int rt);
// The low-rank width in 32-wide units (rank + stab_rank rounded up to a multiple of
// 32: the fused kernels take 16-wide tiles in pairs), at most QD_MAX_TILES.
int quant_down_tiles(int r0, int rt);
constexpr int QD_MAX_TILES = 4;
int quant_down_splits(int64_t M, int64_t K, int rt);
size_t quant_down_partial_bytes(int64_t M, int64_t K, int r0, int rt);

// LoRA parameter gradients, reductions over the M rows (FourTune §3.2: parameter updates
// only for the adapter):
//   dA[r x K] = GB[:, :r]^T * bf16(X)      dB[N x r] = bf16(G)^T * XL[:, :r]
// Split over M; each split writes fp32 partials, summed afterwards in a fixed order
// (deterministic; LoraReduce).
// X and G must each be smaller than 4 GiB (32-bit buffer offsets).
struct LoraGradArgs {
  int64_t M;
  int r;
  // dA job
  const bf16_t* gb;      // [M x rt], first r columns used
  int64_t ld_gb;
  const void* x;         // [M x K] fp32/bf16
  bool x_bf16;
  int64_t K;
  float* dA;             // [r x K]
  // dB job
  const bf16_t* xl;      // [M x rt], first r columns used
  int64_t ld_xl;
  const void* g;         // [M x N] fp32/bf16
  bool g_bf16;
  int64_t N;
  float* dB;             // [N x r]
  // scratch
  float* partials;       // lora_grad_partial_bytes(M, K, N, r) bytes
  bool gelu_x;           // the dA job reads bf16(GELU(x)) instead of bf16(x) (x bf16)
  // set by the launcher
  int tile_offset;
  int ntiles;
};

// With `deferred` non-null the row-range sum is not launched: *deferred describes it
// (items = 0 when there is none), for the caller to hand to the backward GEMM.
hipError_t launch_lora_grad(const LoraGradArgs& a, hipStream_t stream, LoraReduce* deferred = nullptr);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);

// 16-bit activation x 4-bit weight GEMM (precision variants W4A16 / G16):
//   forward : out[M x N] = bf16(act)[M x Kred] deq Q(R)^T + low[M x rt] U^T
//   backward: out[M x N] = bf16(act)[M x Kred] deq Q(R)   + low[M x rt] D
// with Q(R) the linear's weight ([N_lin x K_lin]: forward N = N_lin, Kred = K_lin;
// backward N = K_lin, Kred = N_lin) and U / D split at up_split as in GemmArgs.
struct GemmA16Args {
  const void* act;          // [M x Kred] fp32 or bf16, row stride ld_act
  int64_t ld_act;
  const uint8_t* b_codes;   // Q(R) codes, contiguous rows
  const uint8_t* b_scales;  // Q(R) block scales
  int64_t M, N, Kred;
  const bf16_t* low;        // [M x rt]
  int rt;
  const bf16_t* up0;
  const bf16_t* up1;
  int up_split;
  void* out;                // [M x N] fp32 or bf16, row stride ldo
  int64_t ldo;
};
hipError_t launch_gemm_a16(const GemmA16Args& g, bool act_bf16, bool trans_b, bool out_bf16, hipStream_t stream);

// Unfused pieces for the fusion ablation (the fused path never uses them):
//   out[M x C] = base[M x C] (bf16) + low[M x rt] * V, fp32 accumulation, one rounding
//   forward : V = U^T, U row q = v0[q*r0 .. +r0] ++ v1[q*(rt-r0) .. +(rt-r0)] ([B | L2])
//   backward: V = D,   D row j = v0 row j (j < r0) or v1 row j - r0, row stride C ([A; L1])
// rt a multiple of 32 up to 128, r0 a multiple of 16, C a multiple of 8.
struct UpAddArgs {
  const bf16_t* base;
  const bf16_t* low;
  const bf16_t* v0;
  const bf16_t* v1;
  int64_t M, C;
  int rt, r0;
  void* out;  // fp32 or bf16
};
hipError_t launch_up_add(const UpAddArgs& a, bool bwd, bool out_bf16, hipStream_t stream);
// h = bf16(GELU(p)), dp = bf16(dh * GELU'(p)) over n elements (n a multiple of 8)
hipError_t launch_gelu(const bf16_t* p, bf16_t* h, int64_t n, hipStream_t stream);
hipError_t launch_gelu_bwd(const bf16_t* p, const bf16_t* dh, bf16_t* dp, int64_t n, hipStream_t stream);
int lora_grad_splits(int64_t M, int64_t K, int64_t N, int r);
int lora_grad_tiles(int64_t M, int64_t K, int64_t N, int r);
size_t lora_grad_partial_bytes(int64_t M, int64_t K, int64_t N, int r);

}  // namespace ft
