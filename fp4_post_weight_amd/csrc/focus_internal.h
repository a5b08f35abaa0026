// focus_internal.h -- launchers shared by the kernel file and the C ABI.
// Arguments reaching these functions have been validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace focus {

hipError_t launch_tensor_scale(const uint16_t* w, int64_t numel, float* s2_out, float* amax_out,
                               hipStream_t stream);
hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t cols, const float* m,
                           const float* q, const float* s2, uint8_t* codes, uint8_t* scales,
                           uint16_t* wdeq, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s2,
                             int s2_per_row, int64_t rows, int64_t cols, uint16_t* out,
                             hipStream_t stream);
hipError_t launch_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* codes,
                                uint8_t* scales, float* s2_out, uint16_t* xdeq,
                                hipStream_t stream);

}  // namespace focus
