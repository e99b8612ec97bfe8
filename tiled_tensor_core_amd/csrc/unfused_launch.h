// Internal interface between the C ABI (attn_api.cpp) and the un-fused
// attention kernels (unfused_kernel.hip).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ttc_unf {

struct UnfParams {
  const uint16_t* q;   // [BH, N, D] 16-bit floats
  const uint16_t* k;
  const uint16_t* v;
  float* s;            // workspace: scores, then probabilities, fp32 [BH, N, N]
  float* o;            // [BH, N, D]
  int N;               // sequence length
  float scale;         // multiplier of the scores
};

// Bytes of the device scratch the allocation-free entry point uses for the
// score matrix (B*H*N*N*4 must not exceed it).
constexpr unsigned long long kScratchBytes = 64ull << 20;

// Device address of that scratch on the current device (looked up on the
// first call per device, then cached).
hipError_t scratch_address(void** out);

// Enqueue scores -> row softmax (writing lse) -> P V on `stream`.
// Arguments are already validated (BH <= 65535, BH * N < 2^31).
hipError_t launch_unfused(bool bf16, int d, bool causal, const UnfParams& prm, int BH, float* lse,
                          hipStream_t stream);

}  // namespace ttc_unf
