// C ABI of the W4A4G4 linear layer: argument validation, workspace carving and kernel
// launches on the caller's stream. No allocation, no synchronization, no global
// mutable state besides the thread-local error text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fourtune.h"
#include "launch.h"
#include "gemm.h"

namespace {

thread_local char g_last_error[512] = "";

ft_status fail(ft_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

ft_status ok() {
  g_last_error[0] = '\0';
  return FT_OK;
}

ft_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(ft_dtype d) { return d == FT_F32 ? 4 : 2; }

bool dtype_ok(ft_dtype d) { return d == FT_F32 || d == FT_BF16; }

#define REQUIRE(cond, status, ...)            \
  do {                                        \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define TRY(expr)                         \
  do {                                    \
    ft_status _s = (expr);                \
    if (_s != FT_OK) return _s;           \
  } while (0)

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace carving
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += round_up(bytes, 256);
    return p;
  }
};

ft_status check_mx4(const ft_mx4* t, int64_t rows, int64_t cols, const char* name) {
  REQUIRE(t != nullptr, FT_ERR_NULL, "%s: NULL ft_mx4", name);
  REQUIRE(t->codes && t->scales, FT_ERR_NULL, "%s: NULL codes/scales", name);
  REQUIRE(t->rows == rows && t->cols == cols, FT_ERR_SHAPE,
          "%s: is [%lld x %lld], expected [%lld x %lld]", name, (long long)t->rows,
          (long long)t->cols, (long long)rows, (long long)cols);
  REQUIRE(aligned16(t->codes), FT_ERR_ALIGN, "%s: codes not 16-byte aligned", name);
  return FT_OK;
}

}  // namespace

extern "C" {

size_t ft_mx4_codes_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (size_t)rows * (size_t)(cols / 2);
}

size_t ft_mx4_scales_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (size_t)((rows + 31) / 32) * (size_t)(cols / 32);
}

const char* fourtune_status_string(ft_status s) {
  switch (s) {
    case FT_OK: return "ok";
    case FT_ERR_NULL: return "null pointer";
    case FT_ERR_SHAPE: return "bad shape";
    case FT_ERR_DTYPE: return "bad dtype";
    case FT_ERR_ALIGN: return "misaligned pointer";
    case FT_ERR_WORKSPACE: return "workspace too small";
    case FT_ERR_UNSUPPORTED: return "unsupported";
    case FT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fourtune_last_error(void) { return g_last_error; }

ft_status fourtune_quantize(const void* x, ft_dtype x_dt, int64_t rows, int64_t cols, int64_t ld,
                            ft_mx4* out, void* stream) {
  REQUIRE(dtype_ok(x_dt), FT_ERR_DTYPE, "quantize: unknown dtype %d", (int)x_dt);
  REQUIRE(rows >= 0 && cols >= 0, FT_ERR_SHAPE, "quantize: negative size");
  REQUIRE(cols % 32 == 0, FT_ERR_SHAPE, "quantize: cols=%lld not a multiple of 32", (long long)cols);
  REQUIRE(ld >= cols, FT_ERR_SHAPE, "quantize: ld=%lld < cols=%lld", (long long)ld, (long long)cols);
  REQUIRE((ld * (int64_t)elem_size(x_dt)) % 16 == 0, FT_ERR_ALIGN,
          "quantize: row stride of %lld bytes not a multiple of 16", (long long)(ld * elem_size(x_dt)));
  REQUIRE(rows < (int64_t)65535 * 32, FT_ERR_UNSUPPORTED, "quantize: rows=%lld too large", (long long)rows);
  if (rows == 0 || cols == 0) return ok();
  REQUIRE(x != nullptr, FT_ERR_NULL, "quantize: NULL x");
  REQUIRE(aligned16(x), FT_ERR_ALIGN, "quantize: x not 16-byte aligned");
  TRY(check_mx4(out, rows, cols, "quantize: out"));
  TRY(hip_check(ft::launch_quantize(x, x_dt == FT_BF16, rows, cols, ld, out->codes, out->scales,
                                    static_cast<hipStream_t>(stream)),
                "quantize launch"));
  return ok();
}

ft_status fourtune_quantize_groups(const void* x, ft_dtype x_dt, int64_t rows, int64_t cols, int64_t ld,
                                   ft_mx4* out, void* stream) {
  REQUIRE(dtype_ok(x_dt), FT_ERR_DTYPE, "quantize_groups: unknown dtype %d", (int)x_dt);
  REQUIRE(rows >= 0 && cols >= 0, FT_ERR_SHAPE, "quantize_groups: negative size");
  REQUIRE(cols % 32 == 0, FT_ERR_SHAPE, "quantize_groups: cols=%lld not a multiple of 32", (long long)cols);
  REQUIRE(ld >= cols, FT_ERR_SHAPE, "quantize_groups: ld=%lld < cols=%lld", (long long)ld, (long long)cols);
  REQUIRE((ld * (int64_t)elem_size(x_dt)) % 16 == 0, FT_ERR_ALIGN,
          "quantize_groups: row stride of %lld bytes not a multiple of 16", (long long)(ld * elem_size(x_dt)));
  REQUIRE(rows < (int64_t)65535 * 32, FT_ERR_UNSUPPORTED, "quantize_groups: rows=%lld too large", (long long)rows);
  if (rows == 0 || cols == 0) return ok();
  REQUIRE(x != nullptr, FT_ERR_NULL, "quantize_groups: NULL x");
  REQUIRE(aligned16(x), FT_ERR_ALIGN, "quantize_groups: x not 16-byte aligned");
  TRY(check_mx4(out, rows, cols, "quantize_groups: out"));
  TRY(hip_check(ft::launch_quantize(x, x_dt == FT_BF16, rows, cols, ld, out->codes, out->scales,
                                    static_cast<hipStream_t>(stream), true),
                "quantize_groups launch"));
  return ok();
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- linear helpers
ft_status check_linear(const ft_linear* L, const char* who) {
  REQUIRE(L != nullptr, FT_ERR_NULL, "%s: NULL ft_linear", who);
  REQUIRE(L->n > 0 && L->k > 0 && L->n % 32 == 0 && L->k % 32 == 0, FT_ERR_SHAPE,
          "%s: n=%lld, k=%lld must be positive multiples of 32", who, (long long)L->n, (long long)L->k);
  REQUIRE(L->rank >= 0 && L->stab_rank >= 0 && L->rank % 16 == 0 && L->stab_rank % 16 == 0,
          FT_ERR_SHAPE, "%s: rank=%lld, stab_rank=%lld must be multiples of 16", who,
          (long long)L->rank, (long long)L->stab_rank);
  const int64_t rt = L->rank + L->stab_rank;
  REQUIRE(rt <= 128 && ft::quant_down_tiles((int)L->rank, (int)rt) <= ft::QD_MAX_TILES, FT_ERR_UNSUPPORTED,
          "%s: rank + stab_rank = %lld > 128", who, (long long)rt);
  REQUIRE(L->n <= ft::GEMM_MAX_KRED && L->k <= ft::GEMM_MAX_KRED, FT_ERR_UNSUPPORTED,
          "%s: n=%lld, k=%lld; the 4-bit GEMMs reduce over at most %lld elements", who,
          (long long)L->n, (long long)L->k, (long long)ft::GEMM_MAX_KRED);
  TRY(check_mx4(&L->r, L->n, L->k, "linear: Q(R)"));
  if (L->rank > 0) {
    REQUIRE(L->lora_a && L->lora_b, FT_ERR_NULL, "%s: NULL LoRA factor", who);
    REQUIRE(aligned16(L->lora_a) && aligned16(L->lora_b), FT_ERR_ALIGN, "%s: LoRA factor misaligned", who);
  }
  if (L->stab_rank > 0) {
    REQUIRE(L->stab_down && L->stab_up, FT_ERR_NULL, "%s: NULL stabilizer factor", who);
    REQUIRE(aligned16(L->stab_down) && aligned16(L->stab_up), FT_ERR_ALIGN, "%s: stabilizer factor misaligned", who);
  }
  return FT_OK;
}

ft_status check_tensor(const void* p, const char* who, const char* name) {
  REQUIRE(p != nullptr, FT_ERR_NULL, "%s: NULL %s", who, name);
  REQUIRE(aligned16(p), FT_ERR_ALIGN, "%s: %s not 16-byte aligned", who, name);
  return FT_OK;
}

// An empty batch (m = 0) reads nothing; its LoRA gradients dA [rank x k] and
// dB [n x rank] are zero and are written as such.
ft_status zero_lora_grads(const ft_linear* L, float* d_a, float* d_b, void* stream, const char* who) {
  if (L->rank == 0) return FT_OK;
  TRY(check_tensor(d_a, who, "d_lora_a"));
  TRY(check_tensor(d_b, who, "d_lora_b"));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(hip_check(ft::launch_fill_zero(d_a, L->rank * L->k, st), who));
  return hip_check(ft::launch_fill_zero(d_b, L->n * L->rank, st), who);
}

// Workspace: the call's scratch (Q(X) or Q(dY) when the caller does not take them,
// GB, fp32 partial sums of the split reductions). Nothing in it outlives a call.
struct FwdLayout {
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* partials;
  size_t bytes;
};

FwdLayout fwd_layout(void* ws, int64_t m, const ft_linear* L, bool need_xq) {
  Carver c(ws);
  FwdLayout f{};
  const int rt = (int)(L->rank + L->stab_rank);
  if (need_xq) {
    f.xq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, L->k));
    f.xq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, L->k));
  }
  f.partials = c.take<float>(ft::quant_down_partial_bytes(m, L->k, (int)L->rank, rt));
  f.bytes = c.used;
  return f;
}

struct BwdLayout {
  uint8_t* gq_codes;
  uint8_t* gq_scales;
  ft::bf16_t* GB;
  float* partials;  // quant_down's, then lora_grad's (the kernels run in turn)
  ft::bf16_t* ut;   // [B | L2] transposed, where the wide-operand kernel runs (else null)
  size_t bytes;
};

BwdLayout bwd_layout(void* ws, int64_t m, const ft_linear* L, bool need_gq) {
  Carver c(ws);
  BwdLayout b{};
  const int rt = (int)(L->rank + L->stab_rank);
  if (need_gq) {
    b.gq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, L->n));
    b.gq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, L->n));
  }
  b.GB = c.take<ft::bf16_t>((size_t)m * rt * 2);
  const size_t pq = ft::quant_down_partial_bytes(m, L->n, (int)L->rank, rt);
  const size_t pl = ft::lora_grad_partial_bytes(m, L->k, L->n, (int)L->rank);
  b.partials = c.take<float>(pq > pl ? pq : pl);
  const size_t ub = ft::quant_down_ut_bytes(m, L->n, rt);
  b.ut = ub ? c.take<ft::bf16_t>(ub) : nullptr;
  b.bytes = c.used;
  return b;
}

// Buffer-resource addressing is 32-bit: every activation-sized tensor stays below 4 GiB.
ft_status check_m(int64_t m, const ft_linear* L, const char* who) {
  const int64_t widest = L->n > L->k ? L->n : L->k;
  // 64 rows of margin: offsets of rows just past m must not wrap around
  REQUIRE(m + 64 <= (int64_t)(0xFFFFFF00ull / 4 / (uint64_t)widest), FT_ERR_UNSUPPORTED,
          "%s: m=%lld rows of %lld fp32 elements exceed 4 GiB", who, (long long)m, (long long)widest);
  return FT_OK;
}

// Epilogue options of the 4-bit GEMMs (the MLP's FC2 backward).
struct Epi {
  int kind = ft::GEMM_EPI_NONE;
  const void* pre = nullptr;
  uint8_t* q_codes = nullptr;
  uint8_t* q_scales = nullptr;
  float* dbg = nullptr;
};

ft_status run_gemm_fwd(const ft_linear* L, const uint8_t* xq_codes, const uint8_t* xq_scales,
                       const void* xl, int64_t m, void* y, ft_dtype y_dt, hipStream_t st,
                       const Epi& e = Epi()) {
  ft::GemmArgs g{};
  g.a_codes = xq_codes; g.a_scales = xq_scales;
  g.b_codes = L->r.codes; g.b_scales = L->r.scales; g.b_pitch = L->k / 2;
  g.M = m; g.N = L->n; g.Kred = L->k;
  g.low = static_cast<const ft::bf16_t*>(xl); g.rt = (int)(L->rank + L->stab_rank);
  g.up0 = static_cast<const ft::bf16_t*>(L->lora_b); g.up0_ld = L->rank;
  g.up1 = static_cast<const ft::bf16_t*>(L->stab_up); g.up1_ld = L->stab_rank;
  g.up_split = (int)L->rank;
  g.out = y; g.ldo = L->n;
  g.epi = e.kind; g.pre = static_cast<const ft::bf16_t*>(e.pre); g.q_codes = e.q_codes; g.q_scales = e.q_scales;
  return hip_check(ft::launch_gemm_mx4(g, false, y_dt == FT_BF16, st), "gemm_fwd");
}

ft_status run_gemm_bwd(const ft_linear* L, const uint8_t* gq_codes, const uint8_t* gq_scales,
                       const void* gb, int64_t m, void* dx, ft_dtype dx_dt, hipStream_t st,
                       const Epi& e = Epi(), const ft::LoraReduce& tail = ft::LoraReduce{}) {
  ft::GemmArgs g{};
  g.a_codes = gq_codes; g.a_scales = gq_scales;
  g.b_codes = L->r.codes; g.b_scales = L->r.scales; g.b_pitch = L->k / 2;
  g.M = m; g.N = L->k; g.Kred = L->n;
  g.low = static_cast<const ft::bf16_t*>(gb); g.rt = (int)(L->rank + L->stab_rank);
  g.up0 = static_cast<const ft::bf16_t*>(L->lora_a); g.up0_ld = L->k;
  g.up1 = static_cast<const ft::bf16_t*>(L->stab_down); g.up1_ld = L->k;
  g.up_split = (int)L->rank;
  g.out = dx; g.ldo = L->k;
  g.epi = e.kind; g.pre = static_cast<const ft::bf16_t*>(e.pre); g.q_codes = e.q_codes; g.q_scales = e.q_scales;
  g.dbg = e.dbg;
  g.tail = tail;
  return hip_check(ft::launch_gemm_mx4(g, true, dx_dt == FT_BF16, st), "gemm_bwd");
}

// The fused quantize / down-projection kernel on the rows of x [m x cols] (row stride
// cols). down = true reads the linear's [A; L1] rows (input side), false its
// [B | L2] (output side).
ft_status run_quant_down(int mode, const ft_linear* L, bool down, const void* x, bool x_bf16, int64_t m,
                         int64_t cols, uint8_t* codes, uint8_t* scales, void* low, float* partials,
                         hipStream_t st, const char* what, float* hdbg = nullptr, ft::bf16_t* ut = nullptr) {
  ft::QuantDownArgs qd{};
  qd.mode = mode;
  qd.x = x; qd.M = m; qd.K = cols; qd.ldx = cols;
  qd.codes = codes; qd.scales = scales;
  qd.d0 = static_cast<const ft::bf16_t*>(down ? L->lora_a : L->lora_b);
  qd.d1 = static_cast<const ft::bf16_t*>(down ? L->stab_down : L->stab_up);
  qd.r0 = (int)L->rank; qd.rt = (int)(L->rank + L->stab_rank); qd.u_cols = !down;
  qd.low = static_cast<ft::bf16_t*>(low);
  qd.partials = partials;
  qd.hdbg = hdbg;
  qd.ut = ut;
  return hip_check(ft::launch_quant_down(qd, x_bf16, st), what);
}

size_t qd_partials(int64_t m, int64_t cols, const ft_linear* L) {
  return ft::quant_down_partial_bytes(m, cols, (int)L->rank, (int)(L->rank + L->stab_rank));
}

size_t lg_partials(int64_t m, const ft_linear* L) {
  return ft::lora_grad_partial_bytes(m, L->k, L->n, (int)L->rank);
}

// LoRA gradients of one linear: dA = GB_A^T bf16(x) (or bf16(GELU(x))), dB = bf16(g)^T XL_A.
ft_status run_lora_grad(const ft_linear* L, int64_t m, const void* gb, const void* x, bool x_bf16, bool gelu_x,
                        const void* xl, const void* g, bool g_bf16, float* dA, float* dB, float* partials,
                        hipStream_t st, const char* what, ft::LoraReduce* deferred = nullptr) {
  if (deferred) *deferred = ft::LoraReduce{};
  if (L->rank == 0) return FT_OK;
  const int64_t rt = L->rank + L->stab_rank;
  ft::LoraGradArgs lg{};
  lg.M = m; lg.r = (int)L->rank;
  lg.gb = static_cast<const ft::bf16_t*>(gb); lg.ld_gb = rt; lg.x = x; lg.x_bf16 = x_bf16; lg.K = L->k; lg.dA = dA;
  lg.xl = static_cast<const ft::bf16_t*>(xl); lg.ld_xl = rt; lg.g = g; lg.g_bf16 = g_bf16; lg.N = L->n; lg.dB = dB;
  lg.partials = partials; lg.gelu_x = gelu_x;
  return hip_check(ft::launch_lora_grad(lg, st, deferred), what);
}

// Argument checks of the linear forward (shared by the workspace and scratch forms).
ft_status check_linear_fwd_args(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, const void* y,
                                ft_dtype y_dt, const void* xl_saved, const ft_mx4* xq_out, const char* who) {
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(x_dt) && dtype_ok(y_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) return FT_OK;
  TRY(check_m(m, L, who));
  TRY(check_tensor(x, who, "x"));
  TRY(check_tensor(y, who, "y"));
  if (L->rank + L->stab_rank > 0) TRY(check_tensor(xl_saved, who, "xl_saved"));
  if (xq_out) TRY(check_mx4(xq_out, m, L->k, "linear_fwd: xq_out"));
  return FT_OK;
}

// The forward's two launches: one pass over X (Q(X), XL; fp32 partial sums in
// `partials` when the reduction is split), then the 4-bit GEMM with the up-projection.
ft_status launch_linear_fwd(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, void* y, ft_dtype y_dt,
                            void* xl_saved, uint8_t* xq_codes, uint8_t* xq_scales, float* partials, hipStream_t st) {
  const int64_t rt = L->rank + L->stab_rank;
  ft::QuantDownArgs qd{};
  qd.mode = ft::QD_QUANT;
  qd.x = x; qd.M = m; qd.K = L->k; qd.ldx = L->k;
  qd.codes = xq_codes; qd.scales = xq_scales;
  qd.d0 = static_cast<const ft::bf16_t*>(L->lora_a);
  qd.d1 = static_cast<const ft::bf16_t*>(L->stab_down);
  qd.r0 = (int)L->rank; qd.rt = (int)rt; qd.u_cols = false;
  qd.low = static_cast<ft::bf16_t*>(xl_saved);
  qd.partials = partials;
  TRY(hip_check(ft::launch_quant_down(qd, x_dt == FT_BF16, st), "linear_fwd quant_down"));
  return run_gemm_fwd(L, xq_codes, xq_scales, xl_saved, m, y, y_dt, st);
}

}  // namespace

namespace ft {

ft_status linear_fwd_scratch(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, void* y, ft_dtype y_dt,
                             void* xl_saved, ft_mx4* xq_out, float* scratch, size_t scratch_bytes, void* stream,
                             const char* who) {
  TRY(check_linear_fwd_args(L, x, x_dt, m, y, y_dt, xl_saved, xq_out, who));
  REQUIRE(xq_out != nullptr, FT_ERR_NULL, "%s: xq_out is required (Q(X) is an output here)", who);
  if (m == 0) return ok();
  const size_t need = quant_down_partial_bytes(m, L->k, (int)L->rank, (int)(L->rank + L->stab_rank));
  REQUIRE(need <= scratch_bytes, FT_ERR_UNSUPPORTED,
          "%s: m=%lld, k=%lld, rank + stab_rank=%lld need %zu bytes of scratch, %zu available", who, (long long)m,
          (long long)L->k, (long long)(L->rank + L->stab_rank), need, scratch_bytes);
  TRY(launch_linear_fwd(L, x, x_dt, m, y, y_dt, xl_saved, xq_out->codes, xq_out->scales, scratch,
                        static_cast<hipStream_t>(stream)));
  return ok();
}

ft_status set_error(ft_status s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace ft

extern "C" {

size_t fourtune_linear_workspace_bytes(int64_t m, const ft_linear* L) {
  if (L == nullptr || m < 0) return 0;
  const size_t f = fwd_layout(nullptr, m, L, true).bytes;
  const size_t b = bwd_layout(nullptr, m, L, true).bytes;
  return f > b ? f : b;
}

ft_status fourtune_linear_fwd(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, void* y,
                              ft_dtype y_dt, void* xl_saved, ft_mx4* xq_out, void* ws,
                              size_t ws_bytes, void* stream) {
  const char* who = "linear_fwd";
  TRY(check_linear_fwd_args(L, x, x_dt, m, y, y_dt, xl_saved, xq_out, who));
  if (m == 0) return ok();
  const FwdLayout lay = fwd_layout(ws, m, L, xq_out == nullptr);
  REQUIRE(lay.bytes == 0 || (ws != nullptr && ws_bytes >= lay.bytes), FT_ERR_WORKSPACE,
          "%s: workspace of %zu bytes, %zu needed", who, ws_bytes, lay.bytes);
  if (lay.bytes) REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  uint8_t* xq_codes = xq_out ? xq_out->codes : lay.xq_codes;
  uint8_t* xq_scales = xq_out ? xq_out->scales : lay.xq_scales;
  TRY(launch_linear_fwd(L, x, x_dt, m, y, y_dt, xl_saved, xq_codes, xq_scales, lay.partials,
                        static_cast<hipStream_t>(stream)));
  return ok();
}

ft_status fourtune_linear_bwd(const ft_linear* L, const void* dy, ft_dtype dy_dt, const void* x,
                              ft_dtype x_dt, const void* xl_saved, int64_t m, void* dx,
                              ft_dtype dx_dt, float* d_lora_a, float* d_lora_b, ft_mx4* gq_out,
                              void* ws, size_t ws_bytes, void* stream) {
  const char* who = "linear_bwd";
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(dy_dt) && dtype_ok(x_dt) && dtype_ok(dx_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) {
    TRY(zero_lora_grads(L, d_lora_a, d_lora_b, stream, who));
    return ok();
  }
  TRY(check_m(m, L, who));
  const int64_t rt = L->rank + L->stab_rank;
  TRY(check_tensor(dy, who, "dy"));
  TRY(check_tensor(dx, who, "dx"));
  if (L->rank > 0) {
    TRY(check_tensor(x, who, "x"));
    TRY(check_tensor(xl_saved, who, "xl_saved"));
    TRY(check_tensor(d_lora_a, who, "d_lora_a"));
    TRY(check_tensor(d_lora_b, who, "d_lora_b"));
  }
  if (gq_out) TRY(check_mx4(gq_out, m, L->n, "linear_bwd: gq_out"));
  const BwdLayout lay = bwd_layout(ws, m, L, gq_out == nullptr);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE,
          "%s: workspace of %zu bytes, %zu needed", who, ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* gq_codes = gq_out ? gq_out->codes : lay.gq_codes;
  uint8_t* gq_scales = gq_out ? gq_out->scales : lay.gq_scales;

  ft::QuantDownArgs qd{};
  qd.mode = ft::QD_QUANT;
  qd.x = dy; qd.M = m; qd.K = L->n; qd.ldx = L->n;
  qd.codes = gq_codes; qd.scales = gq_scales;
  qd.d0 = static_cast<const ft::bf16_t*>(L->lora_b);
  qd.d1 = static_cast<const ft::bf16_t*>(L->stab_up);
  qd.r0 = (int)L->rank; qd.rt = (int)rt; qd.u_cols = true;
  qd.low = lay.GB;
  qd.partials = lay.partials;
  qd.ut = lay.ut;
  TRY(hip_check(ft::launch_quant_down(qd, dy_dt == FT_BF16, st), "linear_bwd quant_down"));

  // The LoRA gradients go first (they need GB, not dX); their row-range sum then runs
  // as extra workgroups of the transposed GEMM's launch instead of a launch of its own.
  ft::LoraReduce tail{};
  if (L->rank > 0) {
    ft::LoraGradArgs lg{};
    lg.M = m; lg.r = (int)L->rank;
    lg.gb = lay.GB; lg.ld_gb = rt; lg.x = x; lg.x_bf16 = x_dt == FT_BF16; lg.K = L->k; lg.dA = d_lora_a;
    lg.xl = static_cast<const ft::bf16_t*>(xl_saved); lg.ld_xl = rt; lg.g = dy;
    lg.g_bf16 = dy_dt == FT_BF16; lg.N = L->n; lg.dB = d_lora_b;
    lg.partials = lay.partials;
    TRY(hip_check(ft::launch_lora_grad(lg, st, &tail), "linear_bwd lora_grad"));
  }
  TRY(run_gemm_bwd(L, gq_codes, gq_scales, lay.GB, m, dx, dx_dt, st, Epi(), tail));
  return ok();
}

ft_status fourtune_gemm_fwd(const ft_linear* L, const ft_mx4* xq, const void* xl, int64_t m,
                            void* y, ft_dtype y_dt, void* stream) {
  const char* who = "gemm_fwd";
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(y_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) return ok();
  TRY(check_m(m, L, who));
  TRY(check_mx4(xq, m, L->k, "gemm_fwd: xq"));
  if (L->rank + L->stab_rank > 0) TRY(check_tensor(xl, who, "xl"));
  TRY(check_tensor(y, who, "y"));
  TRY(run_gemm_fwd(L, xq->codes, xq->scales, xl, m, y, y_dt, static_cast<hipStream_t>(stream)));
  return ok();
}

ft_status fourtune_gemm_bwd(const ft_linear* L, const ft_mx4* gq, const void* gb, int64_t m,
                            void* dx, ft_dtype dx_dt, void* stream) {
  const char* who = "gemm_bwd";
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(dx_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) return ok();
  TRY(check_m(m, L, who));
  TRY(check_mx4(gq, m, L->n, "gemm_bwd: gq"));
  if (L->rank + L->stab_rank > 0) TRY(check_tensor(gb, who, "gb"));
  TRY(check_tensor(dx, who, "dx"));
  TRY(run_gemm_bwd(L, gq->codes, gq->scales, gb, m, dx, dx_dt, static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

namespace {

struct MlpFwdLayout {
  uint8_t *xq_codes, *xq_scales, *hq_codes, *hq_scales;
  float* partials;
  size_t bytes;
};

MlpFwdLayout mlp_fwd_layout(void* ws, int64_t m, const ft_linear* fc1, const ft_linear* fc2, bool need_hq) {
  Carver c(ws);
  MlpFwdLayout f{};
  const int64_t d = fc1->k, fdim = fc1->n;
  f.xq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, d));
  f.xq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, d));
  if (need_hq) {
    f.hq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, fdim));
    f.hq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, fdim));
  }
  const size_t p1 = qd_partials(m, d, fc1), p2 = qd_partials(m, fdim, fc2);
  f.partials = c.take<float>(p1 > p2 ? p1 : p2);
  f.bytes = c.used;
  return f;
}

struct MlpBwdLayout {
  uint8_t *gq_codes, *gq_scales, *dpq_codes, *dpq_scales;
  ft::bf16_t *gb2, *gb1, *dp;
  float* partials;
  ft::bf16_t* ut;  // fc2's, then fc1's [B | L2] transposed (else null)
  size_t bytes;
};

MlpBwdLayout mlp_bwd_layout(void* ws, int64_t m, const ft_linear* fc1, const ft_linear* fc2, bool need_dpq) {
  Carver c(ws);
  MlpBwdLayout b{};
  const int64_t fdim = fc1->n, dout = fc2->n;
  b.gq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, dout));
  b.gq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, dout));
  b.gb2 = c.take<ft::bf16_t>((size_t)m * (fc2->rank + fc2->stab_rank) * 2);
  b.dp = c.take<ft::bf16_t>((size_t)m * fdim * 2);
  if (need_dpq) {
    b.dpq_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, fdim));
    b.dpq_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, fdim));
  }
  b.gb1 = c.take<ft::bf16_t>((size_t)m * (fc1->rank + fc1->stab_rank) * 2);
  size_t p = qd_partials(m, dout, fc2);
  p = std::max(p, qd_partials(m, fdim, fc1));
  p = std::max(p, lg_partials(m, fc2));
  p = std::max(p, lg_partials(m, fc1));
  b.partials = c.take<float>(p);
  const size_t ub = std::max(ft::quant_down_ut_bytes(m, dout, (int)(fc2->rank + fc2->stab_rank)),
                             ft::quant_down_ut_bytes(m, fdim, (int)(fc1->rank + fc1->stab_rank)));
  b.ut = ub ? c.take<ft::bf16_t>(ub) : nullptr;
  b.bytes = c.used;
  return b;
}

ft_status check_mlp(const ft_linear* fc1, const ft_linear* fc2, int64_t m, const char* who) {
  TRY(check_linear(fc1, who));
  TRY(check_linear(fc2, who));
  REQUIRE(fc1->n == fc2->k, FT_ERR_SHAPE, "%s: fc1 has %lld outputs, fc2 %lld inputs", who,
          (long long)fc1->n, (long long)fc2->k);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m > 0) {
    TRY(check_m(m, fc1, who));
    TRY(check_m(m, fc2, who));
  }
  return FT_OK;
}

}  // namespace

extern "C" {

size_t fourtune_mlp_workspace_bytes(int64_t m, const ft_linear* fc1, const ft_linear* fc2) {
  if (fc1 == nullptr || fc2 == nullptr || m < 0) return 0;
  const size_t f = mlp_fwd_layout(nullptr, m, fc1, fc2, true).bytes;
  const size_t b = mlp_bwd_layout(nullptr, m, fc1, fc2, true).bytes;
  return f > b ? f : b;
}

ft_status fourtune_mlp_fwd(const ft_linear* fc1, const ft_linear* fc2, const void* x, ft_dtype x_dt, int64_t m,
                           void* y, ft_dtype y_dt, void* xl1_saved, void* pre_saved, void* hl2_saved,
                           ft_mx4* hq_out, float* h_debug, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "mlp_fwd";
  TRY(check_mlp(fc1, fc2, m, who));
  REQUIRE(dtype_ok(x_dt) && dtype_ok(y_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  if (m == 0) return ok();
  TRY(check_tensor(x, who, "x"));
  TRY(check_tensor(y, who, "y"));
  TRY(check_tensor(pre_saved, who, "pre_saved"));
  if (fc1->rank + fc1->stab_rank > 0) TRY(check_tensor(xl1_saved, who, "xl1_saved"));
  if (fc2->rank + fc2->stab_rank > 0) TRY(check_tensor(hl2_saved, who, "hl2_saved"));
  if (hq_out) TRY(check_mx4(hq_out, m, fc1->n, "mlp_fwd: hq_out"));
  if (h_debug) REQUIRE(aligned16(h_debug), FT_ERR_ALIGN, "%s: h_debug not 16-byte aligned", who);
  const MlpFwdLayout lay = mlp_fwd_layout(ws, m, fc1, fc2, hq_out == nullptr);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed",
          who, ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t d = fc1->k, fdim = fc1->n;
  uint8_t* hq_codes = hq_out ? hq_out->codes : lay.hq_codes;
  uint8_t* hq_scales = hq_out ? hq_out->scales : lay.hq_scales;

  TRY(run_quant_down(ft::QD_QUANT, fc1, true, x, x_dt == FT_BF16, m, d, lay.xq_codes, lay.xq_scales, xl1_saved,
                     lay.partials, st, "mlp_fwd quant_down(X)"));
  TRY(run_gemm_fwd(fc1, lay.xq_codes, lay.xq_scales, xl1_saved, m, pre_saved, FT_BF16, st));
  TRY(run_quant_down(ft::QD_GELU_QUANT, fc2, true, pre_saved, true, m, fdim, hq_codes, hq_scales, hl2_saved,
                     lay.partials, st, "mlp_fwd gelu_quant_down(P)", h_debug));
  TRY(run_gemm_fwd(fc2, hq_codes, hq_scales, hl2_saved, m, y, y_dt, st));
  return ok();
}

ft_status fourtune_mlp_bwd(const ft_linear* fc1, const ft_linear* fc2, const void* dy, ft_dtype dy_dt,
                           const void* x, ft_dtype x_dt, const void* xl1_saved, const void* pre_saved,
                           const void* hl2_saved, int64_t m, void* dx, ft_dtype dx_dt, float* d_a1, float* d_b1,
                           float* d_a2, float* d_b2, ft_mx4* dpq_out, float* dp_debug, void* ws, size_t ws_bytes,
                           void* stream) {
  const char* who = "mlp_bwd";
  TRY(check_mlp(fc1, fc2, m, who));
  REQUIRE(dtype_ok(dy_dt) && dtype_ok(x_dt) && dtype_ok(dx_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  if (m == 0) {
    TRY(zero_lora_grads(fc1, d_a1, d_b1, stream, who));
    TRY(zero_lora_grads(fc2, d_a2, d_b2, stream, who));
    return ok();
  }
  TRY(check_tensor(dy, who, "dy"));
  TRY(check_tensor(dx, who, "dx"));
  TRY(check_tensor(pre_saved, who, "pre_saved"));
  if (fc1->rank > 0) {
    TRY(check_tensor(x, who, "x"));
    TRY(check_tensor(xl1_saved, who, "xl1_saved"));
    TRY(check_tensor(d_a1, who, "d_a1"));
    TRY(check_tensor(d_b1, who, "d_b1"));
  }
  if (fc2->rank > 0) {
    TRY(check_tensor(hl2_saved, who, "hl2_saved"));
    TRY(check_tensor(d_a2, who, "d_a2"));
    TRY(check_tensor(d_b2, who, "d_b2"));
  }
  if (dpq_out) TRY(check_mx4(dpq_out, m, fc1->n, "mlp_bwd: dpq_out"));
  if (dp_debug) REQUIRE(aligned16(dp_debug), FT_ERR_ALIGN, "%s: dp_debug not 16-byte aligned", who);
  const MlpBwdLayout lay = mlp_bwd_layout(ws, m, fc1, fc2, dpq_out == nullptr);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed",
          who, ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t fdim = fc1->n, dout = fc2->n;
  uint8_t* dpq_codes = dpq_out ? dpq_out->codes : lay.dpq_codes;
  uint8_t* dpq_scales = dpq_out ? dpq_out->scales : lay.dpq_scales;

  TRY(run_quant_down(ft::QD_QUANT, fc2, false, dy, dy_dt == FT_BF16, m, dout, lay.gq_codes, lay.gq_scales,
                     lay.gb2, lay.partials, st, "mlp_bwd quant_down(dY)", nullptr, lay.ut));
  Epi e;
  e.kind = ft::GEMM_EPI_DGELU_Q; e.pre = pre_saved; e.q_codes = dpq_codes; e.q_scales = dpq_scales;
  e.dbg = dp_debug;
  TRY(run_gemm_bwd(fc2, lay.gq_codes, lay.gq_scales, lay.gb2, m, lay.dp, FT_BF16, st, e));
  if (fc1->rank + fc1->stab_rank > 0)
    TRY(run_quant_down(ft::QD_DOWN, fc1, false, lay.dp, true, m, fdim, nullptr, nullptr, lay.gb1, lay.partials, st,
                       "mlp_bwd down(dP)", nullptr, lay.ut));
  // FC2's LoRA gradients after the down-projection of dP (both use the partials
  // scratch; the down-projection's are consumed by its own sum), their row-range sum
  // as extra workgroups of FC1's transposed GEMM
  ft::LoraReduce tail{};
  TRY(run_lora_grad(fc2, m, lay.gb2, pre_saved, true, true, hl2_saved, dy, dy_dt == FT_BF16, d_a2, d_b2,
                    lay.partials, st, "mlp_bwd lora_grad(fc2)", &tail));
  TRY(run_gemm_bwd(fc1, dpq_codes, dpq_scales, lay.gb1, m, dx, dx_dt, st, Epi(), tail));
  TRY(run_lora_grad(fc1, m, lay.gb1, x, x_dt == FT_BF16, false, xl1_saved, lay.dp, true, d_a1, d_b1,
                    lay.partials, st, "mlp_bwd lora_grad(fc1)"));
  return ok();
}

}  // extern "C"

// ================================================================ fusion ablation
// The same layer computed with the fusions taken apart (FourTune §4, "Kernel Fusion
// Breakdown"): each step a launch of its own, its intermediates stored in HBM as bf16.
namespace {

// The linear without its low-rank branches: the 4-bit backbone alone.
ft_linear backbone_only(const ft_linear* L) {
  ft_linear b = *L;
  b.rank = 0;
  b.stab_rank = 0;
  b.lora_a = b.lora_b = b.stab_down = b.stab_up = nullptr;
  return b;
}

// out = base + low [B | L2]^T (forward) or base + low [A; L1] (backward)
ft_status run_up_add(const ft_linear* L, bool bwd, const void* base, const void* low, int64_t m, void* out,
                     ft_dtype out_dt, hipStream_t st, const char* what) {
  ft::UpAddArgs u{};
  u.base = static_cast<const ft::bf16_t*>(base);
  u.low = static_cast<const ft::bf16_t*>(low);
  u.v0 = static_cast<const ft::bf16_t*>(bwd ? L->lora_a : L->lora_b);
  u.v1 = static_cast<const ft::bf16_t*>(bwd ? L->stab_down : L->stab_up);
  u.M = m;
  u.C = bwd ? L->k : L->n;
  u.rt = (int)(L->rank + L->stab_rank);
  u.r0 = (int)L->rank;
  u.out = out;
  return hip_check(ft::launch_up_add(u, bwd, out_dt == FT_BF16, st), what);
}

struct UnfusedLayout {
  uint8_t* q_codes;    // Q(X) or Q(dY)
  uint8_t* q_scales;
  ft::bf16_t* low;     // GB (backward)
  ft::bf16_t* stored;  // the 4-bit product before the up-projection, bf16
  float* partials;
  size_t bytes;
};

UnfusedLayout unfused_layout(void* ws, int64_t m, const ft_linear* L, bool bwd) {
  Carver c(ws);
  UnfusedLayout u{};
  const int64_t rt = L->rank + L->stab_rank;
  const int64_t qcols = bwd ? L->n : L->k, ocols = bwd ? L->k : L->n;
  u.q_codes = c.take<uint8_t>(ft_mx4_codes_bytes(m, qcols));
  u.q_scales = c.take<uint8_t>(ft_mx4_scales_bytes(m, qcols));
  if (bwd) u.low = c.take<ft::bf16_t>((size_t)m * rt * 2);
  if (rt > 0) u.stored = c.take<ft::bf16_t>((size_t)m * ocols * 2);
  size_t p = qd_partials(m, qcols, L);
  if (bwd) p = std::max(p, lg_partials(m, L));
  u.partials = c.take<float>(p);
  u.bytes = c.used;
  return u;
}

size_t linear_ablation_bytes(int64_t m, const ft_linear* L) {
  size_t b = fourtune_linear_workspace_bytes(m, L);
  b = std::max(b, unfused_layout(nullptr, m, L, false).bytes);
  b = std::max(b, unfused_layout(nullptr, m, L, true).bytes);
  return b;
}

}  // namespace

extern "C" {

size_t fourtune_ablation_workspace_bytes(int64_t m, const ft_linear* fc1, const ft_linear* fc2) {
  if (fc1 == nullptr || m < 0) return 0;
  size_t b = linear_ablation_bytes(m, fc1);
  if (fc2 == nullptr) return b;
  b = std::max(b, linear_ablation_bytes(m, fc2));
  return 2 * round_up((size_t)m * fc1->n * 2, 256) + b;
}

ft_status fourtune_linear_fwd_unfused(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, void* y,
                                      ft_dtype y_dt, void* xl_saved, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "linear_fwd_unfused";
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(x_dt) && dtype_ok(y_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) return ok();
  TRY(check_m(m, L, who));
  REQUIRE(m < (int64_t)65535 * 32, FT_ERR_UNSUPPORTED, "%s: m=%lld too large", who, (long long)m);
  const int64_t rt = L->rank + L->stab_rank;
  TRY(check_tensor(x, who, "x"));
  TRY(check_tensor(y, who, "y"));
  if (rt > 0) TRY(check_tensor(xl_saved, who, "xl_saved"));
  const UnfusedLayout lay = unfused_layout(ws, m, L, false);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
          ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ft_linear bb = backbone_only(L);
  TRY(hip_check(ft::launch_quantize(x, x_dt == FT_BF16, m, L->k, L->k, lay.q_codes, lay.q_scales, st),
                "linear_fwd_unfused quantize"));
  if (rt == 0) {
    TRY(run_gemm_fwd(&bb, lay.q_codes, lay.q_scales, nullptr, m, y, y_dt, st));
    return ok();
  }
  TRY(run_quant_down(ft::QD_DOWN, L, true, x, x_dt == FT_BF16, m, L->k, nullptr, nullptr, xl_saved, lay.partials, st,
                     "linear_fwd_unfused down"));
  TRY(run_gemm_fwd(&bb, lay.q_codes, lay.q_scales, nullptr, m, lay.stored, FT_BF16, st));
  TRY(run_up_add(L, false, lay.stored, xl_saved, m, y, y_dt, st, "linear_fwd_unfused up_add"));
  return ok();
}

ft_status fourtune_linear_bwd_unfused(const ft_linear* L, const void* dy, ft_dtype dy_dt, const void* x,
                                      ft_dtype x_dt, const void* xl_saved, int64_t m, void* dx, ft_dtype dx_dt,
                                      float* d_lora_a, float* d_lora_b, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "linear_bwd_unfused";
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(dy_dt) && dtype_ok(x_dt) && dtype_ok(dx_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) {
    TRY(zero_lora_grads(L, d_lora_a, d_lora_b, stream, who));
    return ok();
  }
  TRY(check_m(m, L, who));
  REQUIRE(m < (int64_t)65535 * 32, FT_ERR_UNSUPPORTED, "%s: m=%lld too large", who, (long long)m);
  const int64_t rt = L->rank + L->stab_rank;
  TRY(check_tensor(dy, who, "dy"));
  TRY(check_tensor(dx, who, "dx"));
  if (L->rank > 0) {
    TRY(check_tensor(x, who, "x"));
    TRY(check_tensor(xl_saved, who, "xl_saved"));
    TRY(check_tensor(d_lora_a, who, "d_lora_a"));
    TRY(check_tensor(d_lora_b, who, "d_lora_b"));
  }
  const UnfusedLayout lay = unfused_layout(ws, m, L, true);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
          ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ft_linear bb = backbone_only(L);
  TRY(hip_check(ft::launch_quantize(dy, dy_dt == FT_BF16, m, L->n, L->n, lay.q_codes, lay.q_scales, st),
                "linear_bwd_unfused quantize"));
  if (rt == 0) {
    TRY(run_gemm_bwd(&bb, lay.q_codes, lay.q_scales, nullptr, m, dx, dx_dt, st));
    return ok();
  }
  TRY(run_quant_down(ft::QD_DOWN, L, false, dy, dy_dt == FT_BF16, m, L->n, nullptr, nullptr, lay.low, lay.partials,
                     st, "linear_bwd_unfused down"));
  TRY(run_gemm_bwd(&bb, lay.q_codes, lay.q_scales, nullptr, m, lay.stored, FT_BF16, st));
  TRY(run_up_add(L, true, lay.stored, lay.low, m, dx, dx_dt, st, "linear_bwd_unfused up_add"));
  TRY(run_lora_grad(L, m, lay.low, x, x_dt == FT_BF16, false, xl_saved, dy, dy_dt == FT_BF16, d_lora_a, d_lora_b,
                    lay.partials, st, "linear_bwd_unfused lora_grad"));
  return ok();
}

ft_status fourtune_mlp_fwd_unfused(const ft_linear* fc1, const ft_linear* fc2, int lora_fused, const void* x,
                                   ft_dtype x_dt, int64_t m, void* y, ft_dtype y_dt, void* xl1_saved,
                                   void* pre_saved, void* h_saved, void* hl2_saved, void* ws, size_t ws_bytes,
                                   void* stream) {
  const char* who = "mlp_fwd_unfused";
  TRY(check_mlp(fc1, fc2, m, who));
  if (m == 0) return ok();
  TRY(check_tensor(pre_saved, who, "pre_saved"));
  TRY(check_tensor(h_saved, who, "h_saved"));
  if (lora_fused) {
    TRY(fourtune_linear_fwd(fc1, x, x_dt, m, pre_saved, FT_BF16, xl1_saved, nullptr, ws, ws_bytes, stream));
  } else {
    TRY(fourtune_linear_fwd_unfused(fc1, x, x_dt, m, pre_saved, FT_BF16, xl1_saved, ws, ws_bytes, stream));
  }
  TRY(hip_check(ft::launch_gelu(static_cast<const ft::bf16_t*>(pre_saved), static_cast<ft::bf16_t*>(h_saved),
                                m * fc1->n, static_cast<hipStream_t>(stream)),
                "mlp_fwd_unfused gelu"));
  if (lora_fused) {
    TRY(fourtune_linear_fwd(fc2, h_saved, FT_BF16, m, y, y_dt, hl2_saved, nullptr, ws, ws_bytes, stream));
  } else {
    TRY(fourtune_linear_fwd_unfused(fc2, h_saved, FT_BF16, m, y, y_dt, hl2_saved, ws, ws_bytes, stream));
  }
  return ok();
}

ft_status fourtune_mlp_bwd_unfused(const ft_linear* fc1, const ft_linear* fc2, int lora_fused, const void* dy,
                                   ft_dtype dy_dt, const void* x, ft_dtype x_dt, const void* xl1_saved,
                                   const void* pre_saved, const void* h_saved, const void* hl2_saved, int64_t m,
                                   void* dx, ft_dtype dx_dt, float* d_a1, float* d_b1, float* d_a2, float* d_b2,
                                   void* ws, size_t ws_bytes, void* stream) {
  const char* who = "mlp_bwd_unfused";
  TRY(check_mlp(fc1, fc2, m, who));
  if (m == 0) {
    TRY(zero_lora_grads(fc1, d_a1, d_b1, stream, who));
    TRY(zero_lora_grads(fc2, d_a2, d_b2, stream, who));
    return ok();
  }
  TRY(check_tensor(pre_saved, who, "pre_saved"));
  TRY(check_tensor(h_saved, who, "h_saved"));
  REQUIRE(ws != nullptr && aligned16(ws), FT_ERR_WORKSPACE, "%s: workspace missing or misaligned", who);
  const size_t inter = round_up((size_t)m * fc1->n * 2, 256);
  REQUIRE(ws_bytes >= 2 * inter, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, more than %zu needed", who,
          ws_bytes, 2 * inter);
  Carver c(ws);
  ft::bf16_t* dh = c.take<ft::bf16_t>(inter);
  ft::bf16_t* dp = c.take<ft::bf16_t>(inter);
  void* rest = static_cast<char*>(ws) + c.used;
  const size_t rest_bytes = ws_bytes - c.used;
  if (lora_fused) {
    TRY(fourtune_linear_bwd(fc2, dy, dy_dt, h_saved, FT_BF16, hl2_saved, m, dh, FT_BF16, d_a2, d_b2, nullptr, rest,
                            rest_bytes, stream));
  } else {
    TRY(fourtune_linear_bwd_unfused(fc2, dy, dy_dt, h_saved, FT_BF16, hl2_saved, m, dh, FT_BF16, d_a2, d_b2, rest,
                                    rest_bytes, stream));
  }
  TRY(hip_check(ft::launch_gelu_bwd(static_cast<const ft::bf16_t*>(pre_saved), dh, dp, m * fc1->n,
                                    static_cast<hipStream_t>(stream)),
                "mlp_bwd_unfused gelu_bwd"));
  if (lora_fused) {
    TRY(fourtune_linear_bwd(fc1, dp, FT_BF16, x, x_dt, xl1_saved, m, dx, dx_dt, d_a1, d_b1, nullptr, rest,
                            rest_bytes, stream));
  } else {
    TRY(fourtune_linear_bwd_unfused(fc1, dp, FT_BF16, x, x_dt, xl1_saved, m, dx, dx_dt, d_a1, d_b1, rest, rest_bytes,
                                    stream));
  }
  return ok();
}

}  // extern "C"

// ================================================================ precision variants
// FourTune §4 "Impact of Precision Configurations": the same layer with the activations
// (A16) and/or the gradients (G16) kept in 16 bits (bf16) while the weight stays 4-bit.
namespace {

ft_status run_gemm_a16(const ft_linear* L, bool bwd, const void* act, ft_dtype act_dt, const void* low, int64_t m,
                       void* out, ft_dtype out_dt, hipStream_t st, const char* what) {
  ft::GemmA16Args g{};
  g.act = act;
  g.ld_act = bwd ? L->n : L->k;
  g.b_codes = L->r.codes;
  g.b_scales = L->r.scales;
  g.M = m;
  g.N = bwd ? L->k : L->n;
  g.Kred = bwd ? L->n : L->k;
  g.low = static_cast<const ft::bf16_t*>(low);
  g.rt = (int)(L->rank + L->stab_rank);
  g.up0 = static_cast<const ft::bf16_t*>(bwd ? L->lora_a : L->lora_b);
  g.up1 = static_cast<const ft::bf16_t*>(bwd ? L->stab_down : L->stab_up);
  g.up_split = (int)L->rank;
  g.out = out;
  g.ldo = g.N;
  return hip_check(ft::launch_gemm_a16(g, act_dt == FT_BF16, bwd, out_dt == FT_BF16, st), what);
}

}  // namespace

extern "C" {

ft_status fourtune_linear_fwd_prec(const ft_linear* L, int prec, const void* x, ft_dtype x_dt, int64_t m, void* y,
                                   ft_dtype y_dt, void* xl_saved, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "linear_fwd_prec";
  REQUIRE(prec >= FT_PREC_W4A4G4 && prec <= FT_PREC_W4A16G16, FT_ERR_UNSUPPORTED, "%s: unknown precision %d", who,
          prec);
  if (prec == FT_PREC_W4A4G4 || prec == FT_PREC_W4A4G16)
    return fourtune_linear_fwd(L, x, x_dt, m, y, y_dt, xl_saved, nullptr, ws, ws_bytes, stream);
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(x_dt) && dtype_ok(y_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) return ok();
  TRY(check_m(m, L, who));
  REQUIRE(m < (int64_t)65535 * 128, FT_ERR_UNSUPPORTED, "%s: m=%lld too large", who, (long long)m);
  const int64_t rt = L->rank + L->stab_rank;
  TRY(check_tensor(x, who, "x"));
  TRY(check_tensor(y, who, "y"));
  if (rt > 0) TRY(check_tensor(xl_saved, who, "xl_saved"));
  const FwdLayout lay = fwd_layout(ws, m, L, false);
  REQUIRE(lay.bytes == 0 || (ws != nullptr && ws_bytes >= lay.bytes), FT_ERR_WORKSPACE,
          "%s: workspace of %zu bytes, %zu needed", who, ws_bytes, lay.bytes);
  if (lay.bytes) REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rt > 0)
    TRY(run_quant_down(ft::QD_DOWN, L, true, x, x_dt == FT_BF16, m, L->k, nullptr, nullptr, xl_saved, lay.partials,
                       st, "linear_fwd_prec down"));
  TRY(run_gemm_a16(L, false, x, x_dt, xl_saved, m, y, y_dt, st, "linear_fwd_prec gemm_a16"));
  return ok();
}

ft_status fourtune_linear_bwd_prec(const ft_linear* L, int prec, const void* dy, ft_dtype dy_dt, const void* x,
                                   ft_dtype x_dt, const void* xl_saved, int64_t m, void* dx, ft_dtype dx_dt,
                                   float* d_lora_a, float* d_lora_b, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "linear_bwd_prec";
  REQUIRE(prec >= FT_PREC_W4A4G4 && prec <= FT_PREC_W4A16G16, FT_ERR_UNSUPPORTED, "%s: unknown precision %d", who,
          prec);
  if (prec == FT_PREC_W4A4G4 || prec == FT_PREC_W4A16G4)
    return fourtune_linear_bwd(L, dy, dy_dt, x, x_dt, xl_saved, m, dx, dx_dt, d_lora_a, d_lora_b, nullptr, ws,
                               ws_bytes, stream);
  TRY(check_linear(L, who));
  REQUIRE(dtype_ok(dy_dt) && dtype_ok(x_dt) && dtype_ok(dx_dt), FT_ERR_DTYPE, "%s: unknown dtype", who);
  REQUIRE(m >= 0, FT_ERR_SHAPE, "%s: m=%lld < 0", who, (long long)m);
  if (m == 0) {
    TRY(zero_lora_grads(L, d_lora_a, d_lora_b, stream, who));
    return ok();
  }
  TRY(check_m(m, L, who));
  REQUIRE(m < (int64_t)65535 * 128, FT_ERR_UNSUPPORTED, "%s: m=%lld too large", who, (long long)m);
  const int64_t rt = L->rank + L->stab_rank;
  TRY(check_tensor(dy, who, "dy"));
  TRY(check_tensor(dx, who, "dx"));
  if (L->rank > 0) {
    TRY(check_tensor(x, who, "x"));
    TRY(check_tensor(xl_saved, who, "xl_saved"));
    TRY(check_tensor(d_lora_a, who, "d_lora_a"));
    TRY(check_tensor(d_lora_b, who, "d_lora_b"));
  }
  const BwdLayout lay = bwd_layout(ws, m, L, false);
  REQUIRE(ws != nullptr && ws_bytes >= lay.bytes, FT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
          ws_bytes, lay.bytes);
  REQUIRE(aligned16(ws), FT_ERR_ALIGN, "%s: workspace misaligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rt > 0)
    TRY(run_quant_down(ft::QD_DOWN, L, false, dy, dy_dt == FT_BF16, m, L->n, nullptr, nullptr, lay.GB, lay.partials,
                       st, "linear_bwd_prec down"));
  TRY(run_gemm_a16(L, true, dy, dy_dt, lay.GB, m, dx, dx_dt, st, "linear_bwd_prec gemm_a16"));
  TRY(run_lora_grad(L, m, lay.GB, x, x_dt == FT_BF16, false, xl_saved, dy, dy_dt == FT_BF16, d_lora_a, d_lora_b,
                    lay.partials, st, "linear_bwd_prec lora_grad"));
  return ok();
}

}  // extern "C"
