// Host-side launchers of the gfx950 kernels (one per kernel family). Every launcher
// enqueues on `stream` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

// 32x32-block MXFP4 quantizer of a [rows x cols] fp32/bf16 tensor with row stride ld.
hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);

}  // namespace ft
