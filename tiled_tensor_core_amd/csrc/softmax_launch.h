// Internal interface between the C ABI (attn_api.cpp) and the row-softmax
// kernels.
#pragma once
#include <hip/hip_runtime_api.h>

namespace ttc_sm {

// Enqueue the row softmax on `stream`; dtype 0 fp32, 1 bf16, 2 fp16.  lse,
// if not null, receives each row's natural log-sum-exp (fp32, one per row;
// the un-fused attention path uses it).  Arguments are already validated.
hipError_t launch_softmax(int dtype, const void* x, void* y, int rows, int cols, float* lse, hipStream_t stream);

}  // namespace ttc_sm
