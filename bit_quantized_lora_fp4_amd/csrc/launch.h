// Host-side launchers of the gfx950 kernels (one per kernel family). Every launcher
// enqueues on `stream` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fourtune.h"

namespace ft {

// MXFP4 quantizer of a [rows x cols] fp32/bf16 tensor with row stride ld: 32x32 blocks
// (scales [ceil(rows/32) x cols/32]) or, with groups, 1x32 groups (scales [rows x cols/32]).
hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream, bool groups = false);

// The linear forward (fourtune_linear_fwd's validation and launches) with Q(X) written
// to xq_out (required) and the split reduction's fp32 partial sums kept in `scratch`
// (device memory of scratch_bytes bytes) instead of a caller workspace; refuses sizes
// whose partials exceed it. Defined with the C ABI.
ft_status linear_fwd_scratch(const ft_linear* L, const void* x, ft_dtype x_dt, int64_t m, void* y, ft_dtype y_dt,
                             void* xl_saved, ft_mx4* xq_out, float* scratch, size_t scratch_bytes, void* stream,
                             const char* who);
// Records `msg` as this thread's last error and returns s.
ft_status set_error(ft_status s, const char* msg);

}  // namespace ft
