// Internal interface between the softmax C ABI (softmax_api.cpp) and its kernels.
#pragma once
#include <hip/hip_runtime_api.h>

namespace ttc_sm {

// Enqueue the row softmax on `stream`; dtype 0 fp32, 1 bf16, 2 fp16.
// Arguments are already validated.
hipError_t launch_softmax(int dtype, const void* x, void* y, int rows, int cols, hipStream_t stream);

}  // namespace ttc_sm
