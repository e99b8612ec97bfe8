// Internal interface between the C ABI (attn_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ttc {

struct AttnParams {
  const uint16_t* q;   // [BH, N, D] 16-bit floats
  const uint16_t* k;
  const uint16_t* v;
  float* o;            // [BH, N, D]
  float* lse;          // [BH, N]
  int BH;              // batch * heads
  int N;               // sequence length
  int n_qblk;          // query blocks per head (set by the launcher)
  int n_dom;           // head domains, one per XCD (8) or a single one (1) (set by the launcher)
  int n_work;          // workgroups per domain (set by the launcher)
  int grp;             // heads per group in a domain's item order (set by the launcher)
  float c;             // |scale| * log2(e), or log2(e) when scale == 0
  float thr;           // raw-score margin before the running maximum moves (set by the launcher)
  int q_mode;          // 0: use Q; 1: use -Q (negative scale); 2: use 0 (zero scale)
  int prio;            // 1: workgroups set their wave priority by progress; 0: they do not
  float l_max;         // fixed-reference mode: bound on a lane's sum of the 16-bit P before
                       // its item is computed again (set by the launcher)
  float headroom;      // fixed-reference mode: log2 units between the first tile's maximum
                       // and the reference (set by the launcher)
};

// Launch configuration; a field of 0 takes the built-in choice.
struct LaunchCfg {
  int n_dom;    // 1 or 8 head domains
  int n_work;   // persistent workgroups per domain
  int grp;      // heads per group in a domain's item order
  int prio;     // 1 on, 2 off
  int mode;     // exponent reference: 1 fixed per item, 2 running maximum
  int tile;     // 1: 128 query rows per workgroup (4 waves); 2: 256 (8 waves, fixed mode)
};

// Query rows per workgroup of a tile variant (1 or 2).
int block_rows(int tile);

// Compiled resources of one kernel variant on the current device.
struct KernelInfo {
  int rows, waves, vgprs, lds_bytes, scratch_bytes, groups_per_cu;
};
hipError_t kernel_info(bool bf16, int d, bool causal, bool fixed, int tile, KernelInfo& out);

// Fill the launch configuration for prm's shape: fields of cfg that are 0
// get the built-in choice, the others are clamped to what the shape allows.
// prm.BH and prm.N must be set.  Queries the device's occupancy once.
hipError_t resolve_cfg(bool bf16, int d, bool causal, const AttnParams& prm, LaunchCfg& cfg);

// Enqueue the kernel on `stream` with a configuration resolve_cfg filled.
// Arguments are already validated.
hipError_t launch_attn_fwd(bool bf16, int d, bool causal, AttnParams prm, const LaunchCfg& cfg,
                           hipStream_t stream);

}  // namespace ttc
