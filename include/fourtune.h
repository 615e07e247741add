/*
 * fourtune.h -- C ABI of the W4A4G4 quantized linear layer on MI355X (gfx950).
 *
 * Method: "FourTune: Towards Fully 4-Bit Efficient Post-Training for Diffusion
 * Models". Weights, activations and gradients are quantized to 4 bits and the
 * backbone matrix products run in 4 bits (§3, opening paragraph). A linear layer has
 * three branches (§3.1): a frozen 4-bit backbone on the residual R = W - L2 L1, a
 * frozen full-precision low-rank stabilizer (L1, L2) and a trainable LoRA adapter
 * (A, B). Quantization is block-wise with block-local scales so that the backward
 * can read the same 4-bit weight transposed (§3.2). Quantization is fused with the
 * down-projections, and the 4-bit GEMM with the up-projections (§3.3 "LoRA Fusion");
 * in an MLP, GELU is fused with the quantization of FC2's input (§3.3 "MLP Fusion").
 *
 * Conventions for every entry point
 *   - Row-major storage everywhere; nn.Linear layout: W is [out x in], Y = X W^T.
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or synchronizes, keeps no pointer after returning, and holds no
 *     mutable global state. Work is enqueued on `stream` (a hipStream_t; NULL = the
 *     null stream) and completes asynchronously.
 *   - Arguments are validated before anything is launched. On a bad argument the call
 *     returns an FT_ERR_* code, launches nothing and records a message readable with
 *     fourtune_last_error() (thread-local). A launch failure returns FT_ERR_HIP.
 *     Faults inside kernels surface at the caller's next synchronization.
 *   - Outputs are overwritten, never accumulated into.
 *   - Required alignment: 16 bytes for every tensor pointer and for the workspace.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs.
 *
 * MXFP4 tensor format (ft_mx4)
 *   A [rows x cols] tensor is cut into 32x32 blocks (the last block row may be
 *   partial; cols must be a multiple of 32). Each element is an E2M1 code: bit 3 the
 *   sign, bits 0..2 the index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Two codes per byte,
 *   the even column in the low nibble: codes is [rows x cols/2] bytes. Each block has
 *   one E8M0 scale byte e, the value being 2^(e-127): scales is
 *   [ceil(rows/32) x cols/32] bytes, row-major over blocks. A block's exponent is
 *   E = clamp(floor(log2(amax)) - 2, -127, 127) (E = -127 for an all-zero block),
 *   elements are rounded to nearest on the E2M1 grid, ties to the even code,
 *   saturating at 6, the sign kept for values that round to zero. A block holding
 *   a NaN or infinity gets scale byte 0xFF and zero codes.
 */
#ifndef FOURTUNE_H
#define FOURTUNE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype codes are plain 32-bit integers with named values, so any integer a
 * caller passes is a defined value that validation can reject (an out-of-range value
 * held in an enum type would not be). */
typedef int32_t ft_status;
enum {
  FT_OK = 0,
  FT_ERR_NULL = 1,         /* a required pointer is NULL                           */
  FT_ERR_SHAPE = 2,        /* a size is negative, inconsistent or not a multiple   */
  FT_ERR_DTYPE = 3,        /* unknown dtype                                        */
  FT_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned                     */
  FT_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required           */
  FT_ERR_UNSUPPORTED = 6,  /* valid request this build does not handle             */
  FT_ERR_HIP = 7           /* the HIP runtime reported an error                    */
};

typedef int32_t ft_dtype;
enum { FT_F32 = 0, FT_BF16 = 1 };

/* One MXFP4 tensor (see the format above). */
typedef struct {
  uint8_t *codes;   /* [rows x cols/2] bytes                      */
  uint8_t *scales;  /* [ceil(rows/32) x cols/32] E8M0 bytes       */
  int64_t rows;
  int64_t cols;     /* multiple of 32                             */
} ft_mx4;

/* One W4A4G4 linear: Y = Q(X) Q(R)^T + X^ L1^T L2^T + X^ A^T B^T (FourTune §3.1).
 * n = out features, k = in features (multiples of 32). rank = r (LoRA), stab_rank = s;
 * each a multiple of 16 (FT_ERR_SHAPE otherwise); either may be 0 (branch absent).
 * Limits of this build (FT_ERR_UNSUPPORTED beyond them): n, k <= 16384; r + s <= 128;
 * (m + 64) * max(n, k) * 4 bytes below 4 GiB (32-bit buffer addressing). */
typedef struct {
  ft_mx4 r;               /* Q(R), rows = n, cols = k (frozen; from fourtune_quantize) */
  const void *lora_a;     /* A  [rank x k]      bf16, trainable down-projection     */
  const void *lora_b;     /* B  [n x rank]      bf16, trainable up-projection       */
  const void *stab_down;  /* L1 [stab_rank x k] bf16, frozen                        */
  const void *stab_up;    /* L2 [n x stab_rank] bf16, frozen                        */
  int64_t n, k, rank, stab_rank;
} ft_linear;

/* Sizes of the two arrays of an MXFP4 tensor. */
size_t ft_mx4_codes_bytes(int64_t rows, int64_t cols);
size_t ft_mx4_scales_bytes(int64_t rows, int64_t cols);

/* fourtune_quantize -- 32x32-block MXFP4 quantization of a [rows x cols] tensor.
 * Source: FourTune §2.3 (Round(W/s) with a group scale; MXFP4) and §3.2 (block-wise
 * quantization with block-local scales). Used once on each frozen residual R.
 *   x      [rows x cols] fp32 or bf16 (x_dt), row stride ld >= cols elements
 *          (ld * element size must keep rows 16-byte aligned).
 *   out    codes/scales buffers of the sizes above; out->rows/cols must equal
 *          rows/cols.
 * rows >= 0 (0 is a no-op), cols a multiple of 32. */
ft_status fourtune_quantize(const void *x, ft_dtype x_dt, int64_t rows, int64_t cols,
                            int64_t ld, ft_mx4 *out, void *stream);

/* fourtune_quantize_groups -- the 1x32 group form of the quantizer, for comparing
 * granularities (FourTune §4, "Impact of Quantization Granularity": block-wise against
 * group-wise scales). Each row's 32-column groups get a scale of their own, by the same
 * rule as a block (E from the group's amax, E2M1 rounding, NaN/Inf group -> 0xFF and
 * zero codes). Arguments as fourtune_quantize, except that out->scales holds
 * [rows x cols/32] bytes, row-major. The layer's entry points use 32x32 blocks only. */
ft_status fourtune_quantize_groups(const void *x, ft_dtype x_dt, int64_t rows, int64_t cols,
                                   int64_t ld, ft_mx4 *out, void *stream);

/* Workspace bytes needed by fourtune_linear_fwd and fourtune_linear_bwd for m rows.
 * The workspace is device scratch owned by the caller (16-byte aligned, contents
 * irrelevant, overwritten by every call; nothing in it outlives a call). Two calls
 * that overlap in time (different streams) must not share one. */
size_t fourtune_linear_workspace_bytes(int64_t m, const ft_linear *L);

/* fourtune_linear_fwd -- forward of one W4A4G4 linear (FourTune §3.1, §3.3 "LoRA
 * Fusion"). One pass over X writes Q(X) and XL = bf16(X^ [A;L1]^T) (X^ = bf16(X));
 * then the 4-bit GEMM Q(X) Q(R)^T runs with the up-projection XL [B|L2]^T accumulated
 * into the same fp32 accumulators before the single store of Y.
 *   x        [m x k] fp32 or bf16 (x_dt), contiguous.
 *   y        [m x n] fp32 or bf16 (y_dt), overwritten.
 *   xl_saved [m x (rank + stab_rank)] bf16, overwritten; pass it to the backward.
 *   xq_out   optional (may be NULL): receives Q(X) ([m x k] MXFP4) instead of the
 *            workspace holding it.
 *   ws       workspace of fourtune_linear_workspace_bytes(m, L) bytes. */
ft_status fourtune_linear_fwd(const ft_linear *L, const void *x, ft_dtype x_dt, int64_t m,
                              void *y, ft_dtype y_dt, void *xl_saved, ft_mx4 *xq_out,
                              void *ws, size_t ws_bytes, void *stream);

/* fourtune_linear_bwd -- backward of one W4A4G4 linear (FourTune §3.2). The incoming
 * gradient G = dY is quantized in the same 32x32 blocks, in the same pass as
 * GB = bf16(G^ [B|L2]) (G^ = bf16(G)); dX = Q(G) Q(R) + GB [A;L1] is a 4-bit GEMM that
 * reads the forward's Q(R) codes and scales transposed, with no requantization. Only
 * the adapter gets parameter gradients: dA = GB[:, :r]^T X^, dB = G^^T XL[:, :r].
 *   dy        [m x n] fp32 or bf16 (dy_dt).
 *   x         [m x k] the forward's input (x_dt).
 *   xl_saved  [m x (r+s)] bf16 from fourtune_linear_fwd.
 *   dx        [m x k] fp32 or bf16 (dx_dt), overwritten.
 *   d_lora_a  [rank x k] fp32, overwritten (may be NULL only when rank == 0).
 *   d_lora_b  [n x rank] fp32, overwritten (may be NULL only when rank == 0).
 *   gq_out    optional (may be NULL): receives Q(dY) ([m x n] MXFP4).
 *   ws        workspace of fourtune_linear_workspace_bytes(m, L) bytes.
 * m = 0 (an empty batch) reads nothing and sets dA and dB to zero; the same holds for
 * every backward entry point (the MLP's for both linears, the ablation and precision
 * forms). */
ft_status fourtune_linear_bwd(const ft_linear *L, const void *dy, ft_dtype dy_dt,
                              const void *x, ft_dtype x_dt, const void *xl_saved, int64_t m,
                              void *dx, ft_dtype dx_dt, float *d_lora_a, float *d_lora_b,
                              ft_mx4 *gq_out, void *ws, size_t ws_bytes, void *stream);

/* fourtune_gemm_fwd -- the forward's second kernel on its own: given Q(X) and XL
 * (e.g. produced by a previous fused epilogue), Y = Q(X) Q(R)^T + XL [B|L2]^T, the
 * up-projection accumulated with the 4-bit product before the single store of Y
 * (FourTune §3.3 "LoRA Fusion").
 *   xq  Q(X), [m x k] MXFP4.   xl  [m x (rank + stab_rank)] bf16.
 *   y   [m x n] fp32 or bf16 (y_dt), overwritten. No workspace. */
ft_status fourtune_gemm_fwd(const ft_linear *L, const ft_mx4 *xq, const void *xl, int64_t m,
                            void *y, ft_dtype y_dt, void *stream);

/* fourtune_gemm_bwd -- the backward's 4-bit GEMM on its own: given Q(dY) and GB,
 * dX = Q(dY) Q(R) + GB [A;L1], reading Q(R)'s codes and block scales transposed
 * (FourTune §3.2).
 *   gq  Q(dY), [m x n] MXFP4.  gb  [m x (rank + stab_rank)] bf16.
 *   dx  [m x k] fp32 or bf16 (dx_dt), overwritten. No workspace. */
ft_status fourtune_gemm_bwd(const ft_linear *L, const ft_mx4 *gq, const void *gb, int64_t m,
                            void *dx, ft_dtype dx_dt, void *stream);

/* Workspace bytes needed by fourtune_mlp_fwd and fourtune_mlp_bwd for m rows
 * (same contract as the linear's workspace). */
size_t fourtune_mlp_workspace_bytes(int64_t m, const ft_linear *fc1, const ft_linear *fc2);

/* fourtune_mlp_fwd -- FC1 -> GELU (tanh form) -> FC2 (FourTune §3.3 "MLP Fusion").
 * fc1: d -> f, fc2: f -> d (fc1->n == fc2->k). Kernels, in order:
 *   1. one pass over X: Q(X) and XL1 = bf16(X^ [A1;L1_1]^T)            (§3.3 "LoRA Fusion")
 *   2. FC1's 4-bit GEMM + up-projection, storing P^ = bf16(FC1 output)
 *   3. one pass over P^: H = GELU(P^) in fp32, FC2's 4-bit operand Q(H) and
 *      HL2 = bf16(bf16(H) [A2;L1_2]^T); H itself is never written to memory
 *                                                                       (§3.3 "MLP Fusion")
 *   4. FC2's 4-bit GEMM + up-projection: y = Q(H) Q(R2)^T + HL2 [B2|L2_2]^T.
 *   x         [m x d] fp32 or bf16 (x_dt), contiguous
 *   y         [m x fc2->n] fp32 or bf16 (y_dt), overwritten
 *   xl1_saved [m x rt1] bf16, pre_saved [m x f] bf16, hl2_saved [m x rt2] bf16:
 *             overwritten; pass them to the backward.
 *   hq_out    optional (may be NULL): receives Q(H) ([m x f] MXFP4) instead of the
 *             workspace holding it.
 *   h_debug   optional (may be NULL): [m x f] fp32, receives the fp32 H that step 3
 *             quantized (for checking Q(H) bit for bit); costs 4 bytes per element.
 * f must be at most 16384 (it is FC2's reduction length). */
ft_status fourtune_mlp_fwd(const ft_linear *fc1, const ft_linear *fc2, const void *x,
                           ft_dtype x_dt, int64_t m, void *y, ft_dtype y_dt, void *xl1_saved,
                           void *pre_saved, void *hl2_saved, ft_mx4 *hq_out, float *h_debug,
                           void *ws, size_t ws_bytes, void *stream);

/* fourtune_mlp_bwd -- backward of the MLP pair (FourTune §3.2 for each linear, §3.3
 * "MLP Fusion" for the GELU). Kernels, in order:
 *   1. one pass over dY: Q(dY) and GB2 = bf16(dY^ [B2|L2_2])
 *   2. FC2's transposed 4-bit GEMM + up-projection gives dH; its epilogue forms
 *      dP = dH * GELU'(P^) in fp32, writes Q(dP) (FC1's 4-bit gradient operand) and
 *      stores dP^ = bf16(dP)
 *   3. FC2's LoRA gradients: dA2 = GB2_A^T bf16(GELU(P^)), dB2 = dY^^T HL2_A
 *   4. GB1 = bf16(dP^ [B1|L2_1])
 *   5. FC1's transposed 4-bit GEMM + up-projection: dx = Q(dP) Q(R1) + GB1 [A1;L1_1]
 *   6. FC1's LoRA gradients: dA1 = GB1_A^T X^, dB1 = dP^^T XL1_A.
 *   dy [m x fc2->n] (dy_dt); x, xl1_saved, pre_saved, hl2_saved from the forward;
 *   dx [m x d] (dx_dt), overwritten; d_a1 [r1 x d], d_b1 [f x r1], d_a2 [r2 x f],
 *   d_b2 [fc2->n x r2] fp32, overwritten (may be NULL when that rank is 0).
 *   dpq_out optional (may be NULL): receives Q(dP) ([m x f] MXFP4).
 *   dp_debug optional (may be NULL): [m x f] fp32, receives the fp32 dP that step 2
 *            quantized (for checking Q(dP) bit for bit). */
ft_status fourtune_mlp_bwd(const ft_linear *fc1, const ft_linear *fc2, const void *dy,
                           ft_dtype dy_dt, const void *x, ft_dtype x_dt, const void *xl1_saved,
                           const void *pre_saved, const void *hl2_saved, int64_t m, void *dx,
                           ft_dtype dx_dt, float *d_a1, float *d_b1, float *d_a2, float *d_b2,
                           ft_mx4 *dpq_out, float *dp_debug, void *ws, size_t ws_bytes,
                           void *stream);

/* ---------------------------------------------------------------- fusion ablation
 * The same layer with the fusions taken apart, for measuring what they save (FourTune
 * §4, "Kernel Fusion Breakdown", Figure 9: LoRA fusion over the unfused 4-bit
 * baseline, then MLP fusion on top). Every step is a launch of its own and every
 * intermediate goes through HBM in bf16:
 *   linear forward : Q(X) (quantizer); XL = bf16(X^ [A;L1]^T) (down-projection alone);
 *                    Y0 = bf16(Q(X) Q(R)^T) (4-bit GEMM alone);
 *                    y = Y0 + XL [B|L2]^T (up-projection + add, one rounding)
 *   linear backward: Q(dY); GB = bf16(dY^ [B|L2]); dX0 = bf16(Q(dY) Q(R));
 *                    dx = dX0 + GB [A;L1]; dA, dB as in fourtune_linear_bwd
 *   MLP            : H = bf16(GELU(P^)) stored and fed to FC2 (so FC2's 4-bit operand
 *                    is Q(H) of the bf16 H); backward dH stored in bf16, then
 *                    dP^ = bf16(dH GELU'(P^)) in its own pass.
 * The results differ from the fused entry points only by those bf16 roundings.
 * Arguments are those of the fused entry points; the workspace is
 * fourtune_ablation_workspace_bytes(m, fc1, fc2) bytes (fc2 = NULL for one linear).
 * lora_fused != 0 builds the MLP from the fused linears (fourtune_linear_fwd/bwd) with
 * GELU still separate; 0 from the unfused ones. h_saved [m x f] bf16 receives H in the
 * forward and is read by the backward. */
size_t fourtune_ablation_workspace_bytes(int64_t m, const ft_linear *fc1, const ft_linear *fc2);
ft_status fourtune_linear_fwd_unfused(const ft_linear *L, const void *x, ft_dtype x_dt, int64_t m,
                                      void *y, ft_dtype y_dt, void *xl_saved, void *ws,
                                      size_t ws_bytes, void *stream);
ft_status fourtune_linear_bwd_unfused(const ft_linear *L, const void *dy, ft_dtype dy_dt,
                                      const void *x, ft_dtype x_dt, const void *xl_saved,
                                      int64_t m, void *dx, ft_dtype dx_dt, float *d_lora_a,
                                      float *d_lora_b, void *ws, size_t ws_bytes, void *stream);
ft_status fourtune_mlp_fwd_unfused(const ft_linear *fc1, const ft_linear *fc2, int lora_fused,
                                   const void *x, ft_dtype x_dt, int64_t m, void *y,
                                   ft_dtype y_dt, void *xl1_saved, void *pre_saved,
                                   void *h_saved, void *hl2_saved, void *ws, size_t ws_bytes,
                                   void *stream);
ft_status fourtune_mlp_bwd_unfused(const ft_linear *fc1, const ft_linear *fc2, int lora_fused,
                                   const void *dy, ft_dtype dy_dt, const void *x, ft_dtype x_dt,
                                   const void *xl1_saved, const void *pre_saved,
                                   const void *h_saved, const void *hl2_saved, int64_t m,
                                   void *dx, ft_dtype dx_dt, float *d_a1, float *d_b1,
                                   float *d_a2, float *d_b2, void *ws, size_t ws_bytes,
                                   void *stream);

/* ---------------------------------------------------------------- precision variants
 * FourTune §4 "Impact of Precision Configurations": W4A4G4 (the layer above), W4A16G4,
 * W4A4G16 and W4A16G16. A16 keeps the activation X (as bf16(X)) instead of Q(X) in
 * the forward's backbone product, G16 keeps bf16(dY) instead of Q(dY) in the
 * backward's; the weight is Q(R) in every configuration. The 16-bit products run as
 * bf16 MFMA on the weight dequantized exactly to bf16 as it is staged (only W4A4G4
 * uses the 4-bit matrix cores); the low-rank branches, the LoRA gradients and the
 * saved XL are as in fourtune_linear_fwd / _bwd, whose arguments and workspace
 * (fourtune_linear_workspace_bytes) these take, plus `prec` (an ft_prec value). */
typedef enum {
  FT_PREC_W4A4G4 = 0,
  FT_PREC_W4A16G4 = 1,
  FT_PREC_W4A4G16 = 2,
  FT_PREC_W4A16G16 = 3
} ft_prec;
ft_status fourtune_linear_fwd_prec(const ft_linear *L, int prec, const void *x, ft_dtype x_dt,
                                   int64_t m, void *y, ft_dtype y_dt, void *xl_saved, void *ws,
                                   size_t ws_bytes, void *stream);
ft_status fourtune_linear_bwd_prec(const ft_linear *L, int prec, const void *dy, ft_dtype dy_dt,
                                   const void *x, ft_dtype x_dt, const void *xl_saved, int64_t m,
                                   void *dx, ft_dtype dx_dt, float *d_lora_a, float *d_lora_b,
                                   void *ws, size_t ws_bytes, void *stream);

/* fourtune_linear_fwd_noalloc -- fourtune_linear_fwd for callers that cannot allocate
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, and the library allocates nothing. Q(X) is an
 * output here, so xq_out is required ([m x k] MXFP4); the split reduction's fp32
 * partial sums live in a device array inside the library, 24 MiB per GPU, held until
 * the process ends. Results equal fourtune_linear_fwd's bit for bit. Sizes whose
 * partial sums exceed 24 MiB return FT_ERR_UNSUPPORTED (with rank + stab_rank <= 128
 * none do: at most 16 MiB).
 * Calls that overlap in time on one GPU (different streams, threads) share the array
 * and race: serialize them. Other arguments and errors as fourtune_linear_fwd. */
ft_status fourtune_linear_fwd_noalloc(const ft_linear *L, const void *x, ft_dtype x_dt, int64_t m,
                                      void *y, ft_dtype y_dt, void *xl_saved, ft_mx4 *xq_out,
                                      void *stream);

/* Static text of a status code. */
const char *fourtune_status_string(ft_status s);
/* Detail of the last failing call on this thread ("" if none). */
const char *fourtune_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FOURTUNE_H */
