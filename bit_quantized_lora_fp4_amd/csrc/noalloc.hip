// fourtune_linear_fwd_noalloc: the linear forward for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The only scratch the forward needs beyond its inputs and outputs is the fp32 partial
// sums of the split quantize + down-projection reduction; here they live in a
// file-scope device array, one copy per GPU, instead of a caller workspace. Q(X) is an
// output the caller passes. No allocation, no free, no allocating library call.
//
// Size: a split reduction writes S * M * (rank + stab_rank) floats. S column ranges are
// chosen for about one workgroup per CU (S <= 256 / ceil(M / 64) with 64-row stripes,
// S <= 256 / ceil(M / 128) with the 128-row stripes of the wide-operand kernel), so
// S * M <= 32768 whenever S > 1 and rank + stab_rank <= 128 needs at most 16 MiB; the
// array holds 24 MiB. Every call on one GPU uses that GPU's
// array and overwrites what it uses (nothing must start at zero); calls that overlap
// in time on one GPU race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "fourtune.h"
#include "launch.h"

namespace {

constexpr size_t SCRATCH_BYTES = size_t(24) << 20;
constexpr int MAX_DEVICES = 64;

// In host code `scratch` names a host-side stand-in; the device address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

std::once_flag g_once[MAX_DEVICES];
void* g_scratch[MAX_DEVICES];
hipError_t g_status[MAX_DEVICES];

}  // namespace

extern "C" ft_status fourtune_linear_fwd_noalloc(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m,
                                                 void* y, ft_dtype y_dt, void* xl_saved, ft_mx4* xq_out,
                                                 void* stream) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ft::set_error(FT_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return ft::set_error(FT_ERR_UNSUPPORTED, "linear_fwd_noalloc: device index >= 64");
  std::call_once(g_once[dev], [dev] {
    g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_status[dev] != hipSuccess || g_scratch[dev] == nullptr) {
    char msg[256];
    snprintf(msg, sizeof msg, "linear_fwd_noalloc: hipGetSymbolAddress of the scratch array on device %d: %s", dev,
             hipGetErrorString(g_status[dev]));
    return ft::set_error(FT_ERR_HIP, msg);
  }
  return ft::linear_fwd_scratch(L, x, x_dt, m, y, y_dt, xl_saved, xq_out, static_cast<float*>(g_scratch[dev]),
                                SCRATCH_BYTES, stream, "linear_fwd_noalloc");
}
