// Host-side launchers of the gfx950 kernels (one per kernel family). Every launcher
// enqueues on `stream` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

// MXFP4 quantizer of a [rows x cols] fp32/bf16 tensor with row stride ld: 32x32 blocks
// (scales [ceil(rows/32) x cols/32]) or, with groups, 1x32 groups (scales [rows x cols/32]).
hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream, bool groups = false);

}  // namespace ft
