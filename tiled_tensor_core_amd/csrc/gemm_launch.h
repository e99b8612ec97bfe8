// Internal interface between the C ABI (attn_api.cpp) and the GEMM kernel.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ttc_gemm {

struct GemmParams {
  const uint16_t* a;     // [M, K] bf16, K contiguous
  const uint16_t* w;     // [N, K] bf16, K contiguous
  const float* bias;     // [N] fp32 (unused without a bias epilogue)
  uint16_t* c;           // [M, N] bf16
  int M, N, K;
  int tiles_m, tiles_n;  // set by the launcher
};

// Enqueue C = epilogue(A W^T (+ bias)) on `stream`; epi 0 none, 1 bias,
// 2 bias + GELU.  Arguments are already validated.
hipError_t launch_gemm(int epi, const GemmParams& prm, hipStream_t stream);

}  // namespace ttc_gemm
