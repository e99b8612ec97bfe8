// C ABI of the attention forward pass: argument checks, scale handling and
// dispatch.  Every check runs on the host before any HIP call, so a rejected
// call touches neither the device nor the HIP runtime.

#include <stdint.h>

#include <cmath>
#include <string>

#include "../../include/attn.h"
#include "../../include/gemm.h"
#include "../../include/softmax.h"
#include "attn_launch.h"
#include "gemm_launch.h"
#include "softmax_launch.h"
#include "unfused_launch.h"

namespace {

thread_local std::string g_last_error;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Sizes the kernel can address.  B*H must fit an int; element offsets
// between heads are 64-bit inside the kernel.  Within a head, K, V and O are
// addressed with unsigned 32-bit byte offsets: O is fp32, and the stores of a
// ragged last block of 128 rows compute offsets up to (N + 128) * d * 4.
bool shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return false;
  const long long bh = (long long)B * H;
  const long long rows = bh * N;
  if (bh > (1LL << 30) || rows > (1LL << 40) || rows * d > (1LL << 46)) return false;
  return (long long)(N + 128) * d * 4 <= 0xffffffffLL;
}

// Fields of a caller's launch configuration: 0 (built-in choice) or in range.
bool cfg_valid(const attn_launch_cfg* c, long long bh) {
  if (!c) return true;
  if (c->n_dom != 0 && c->n_dom != 1 && c->n_dom != 8) return false;
  if (c->n_dom == 8 && bh % 8 != 0) return false;
  if (c->n_work < 0 || c->n_work > ATTN_MAX_WORKGROUPS) return false;
  if (c->grp < 0) return false;
  if (c->prio != ATTN_PRIO_DEFAULT && c->prio != ATTN_PRIO_ON && c->prio != ATTN_PRIO_OFF) return false;
  if (c->mode != ATTN_REF_DEFAULT && c->mode != ATTN_REF_FIXED && c->mode != ATTN_REF_RUNNING) return false;
  if (c->tile != ATTN_TILE_DEFAULT && c->tile != ATTN_TILE_128 && c->tile != ATTN_TILE_256) return false;
  if (c->tile == ATTN_TILE_256 && c->mode == ATTN_REF_RUNNING) return false;   // no such kernel
  return true;
}

int run(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N,
        int d, int causal, float scale, void* stream, int dtype, const attn_launch_cfg* user_cfg) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (!shape_ok(B, H, N, d)) return ATTN_ERR_SHAPE;
  const long long bh = (long long)B * H;
  const long long rows = bh * N;
  if (!cfg_valid(user_cfg, bh)) return ATTN_ERR_CONFIG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return ATTN_ERR_ALIGN;
  const size_t in_bytes = (size_t)rows * d * 2, o_bytes = (size_t)rows * d * 4,
               lse_bytes = (size_t)rows * 4;
  if (overlaps(o, o_bytes, lse, lse_bytes) || overlaps(o, o_bytes, q, in_bytes) ||
      overlaps(o, o_bytes, k, in_bytes) || overlaps(o, o_bytes, v, in_bytes) ||
      overlaps(lse, lse_bytes, q, in_bytes) || overlaps(lse, lse_bytes, k, in_bytes) ||
      overlaps(lse, lse_bytes, v, in_bytes))
    return ATTN_ERR_ALIAS;

  ttc::AttnParams prm{};
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.o = o;
  prm.lse = lse;
  prm.BH = (int)bh;
  prm.N = N;
  // The kernel works with a positive score multiplier c = |scale| * log2(e).
  // A negative scale negates Q instead (exact for 16-bit floats), a zero
  // scale zeroes it; either way scale * (q . k) is unchanged.
  const double log2e = 1.4426950408889634074;
  if (scale > 0.0f) {
    prm.c = (float)((double)scale * log2e);
    prm.q_mode = 0;
  } else if (scale < 0.0f) {
    prm.c = (float)(-(double)scale * log2e);
    prm.q_mode = 1;
  } else {
    prm.c = (float)log2e;
    prm.q_mode = 2;
  }
  if (!std::isfinite(prm.c)) return ATTN_ERR_SCALE;  // |scale| * log2(e) overflows fp32
  if (prm.c == 0.0f) {  // |scale| below fp32 range: every score rounds to 0
    prm.c = (float)log2e;
    prm.q_mode = 2;
  }

  ttc::LaunchCfg cfg{};
  if (user_cfg) cfg = {user_cfg->n_dom, user_cfg->n_work, user_cfg->grp, user_cfg->prio, user_cfg->mode, user_cfg->tile};
  hipError_t e = ttc::resolve_cfg(dtype == ATTN_BF16, d, causal == 1, prm, cfg);
  if (e == hipSuccess)
    e = ttc::launch_attn_fwd(dtype == ATTN_BF16, d, causal == 1, prm, cfg, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// Shapes the un-fused path takes: attn_fwd's, with B*H in one grid
// dimension (<= 65535) and B*H*N softmax rows in an int.
bool unfused_shape_ok(int B, int H, int N, int d) {
  if (!shape_ok(B, H, N, d)) return false;
  const long long bh = (long long)B * H;
  return bh <= 65535 && bh * N < (1LL << 31);
}

unsigned long long unfused_ws_bytes(int B, int H, int N) {
  return (unsigned long long)B * (unsigned long long)H * (unsigned long long)N * (unsigned long long)N * 4ull;
}

// ws == nullptr with ws_bytes == 0 and use_scratch: the library's scratch
// (looked up after every host check has passed).
int run_unfused(const void* q, const void* k, const void* v, float* o, float* lse, void* ws,
                unsigned long long ws_bytes, int B, int H, int N, int d, int causal, float scale, void* stream,
                int dtype, bool use_scratch = false) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (!unfused_shape_ok(B, H, N, d)) return ATTN_ERR_SHAPE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse)) return ATTN_ERR_ALIGN;
  const unsigned long long need = unfused_ws_bytes(B, H, N);
  if (use_scratch) {
    if (need > ttc_unf::kScratchBytes) return ATTN_ERR_SCRATCH;
  } else if (!ws || misaligned(ws) || ws_bytes < need) {
    return ATTN_ERR_WORKSPACE;
  }
  const long long rows = (long long)B * H * N;
  const size_t in_bytes = (size_t)rows * d * 2, o_bytes = (size_t)rows * d * 4, lse_bytes = (size_t)rows * 4;
  if (overlaps(o, o_bytes, lse, lse_bytes) || overlaps(o, o_bytes, q, in_bytes) ||
      overlaps(o, o_bytes, k, in_bytes) || overlaps(o, o_bytes, v, in_bytes) ||
      overlaps(lse, lse_bytes, q, in_bytes) || overlaps(lse, lse_bytes, k, in_bytes) ||
      overlaps(lse, lse_bytes, v, in_bytes) || overlaps(ws, need, q, in_bytes) || overlaps(ws, need, k, in_bytes) ||
      overlaps(ws, need, v, in_bytes) || overlaps(ws, need, o, o_bytes) || overlaps(ws, need, lse, lse_bytes))
    return ATTN_ERR_ALIAS;
  if (use_scratch) {
    const hipError_t se = ttc_unf::scratch_address(&ws);
    if (se != hipSuccess) {
      g_last_error = hipGetErrorString(se);
      return ATTN_ERR_HIP;
    }
  }
  ttc_unf::UnfParams prm{};
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.s = static_cast<float*>(ws);
  prm.o = o;
  prm.N = N;
  prm.scale = scale;
  const hipError_t e = ttc_unf::launch_unfused(dtype == ATTN_BF16, d, causal == 1, prm, B * H, lse,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int run_softmax(const void* x, void* y, int rows, int cols, int dtype, void* stream) {
  if (dtype != SOFTMAX_F32 && dtype != SOFTMAX_BF16 && dtype != SOFTMAX_FP16) return ATTN_ERR_DTYPE;
  if (!x || !y) return ATTN_ERR_NULL;
  if (rows < 1 || cols < 1) return ATTN_ERR_SHAPE;
  const long long esize = dtype == SOFTMAX_F32 ? 4 : 2;
  // a row is addressed with 32-bit byte offsets; the matrix with 64-bit ones
  if ((long long)cols * esize > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const long long bytes = (long long)rows * cols * esize;
  if (misaligned(x) || misaligned(y)) return ATTN_ERR_ALIGN;
  if (x != y && overlaps(x, (size_t)bytes, y, (size_t)bytes)) return ATTN_ERR_ALIAS;
  hipError_t e = ttc_sm::launch_softmax(dtype, x, y, rows, cols, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

int run_gemm(const void* a, const void* w, const float* bias, void* c, int M, int N, int K, int epi,
             void* stream) {
  if (epi != GEMM_EPI_NONE && epi != GEMM_EPI_BIAS && epi != GEMM_EPI_BIAS_GELU) return ATTN_ERR_CONFIG;
  if (!a || !w || !c || (epi != GEMM_EPI_NONE && !bias)) return ATTN_ERR_NULL;
  constexpr int kMaxNK = 4194296;   // 256 rows of N or K bf16 values within 2^31 bytes
  if (M < 1 || N < 8 || K < 8 || N % 8 != 0 || K % 8 != 0 || N > kMaxNK || K > kMaxNK)
    return ATTN_ERR_SHAPE;
  if (misaligned(a) || misaligned(w) || misaligned(c) || (bias && misaligned(bias))) return ATTN_ERR_ALIGN;
  const size_t a_bytes = (size_t)M * K * 2, w_bytes = (size_t)N * K * 2, c_bytes = (size_t)M * N * 2;
  if (overlaps(c, c_bytes, a, a_bytes) || overlaps(c, c_bytes, w, w_bytes) ||
      (bias && overlaps(c, c_bytes, bias, (size_t)N * 4)))
    return ATTN_ERR_ALIAS;
  ttc_gemm::GemmParams prm{};
  prm.a = static_cast<const uint16_t*>(a);
  prm.w = static_cast<const uint16_t*>(w);
  prm.bias = bias;
  prm.c = static_cast<uint16_t*>(c);
  prm.M = M;
  prm.N = N;
  prm.K = K;
  hipError_t e = ttc_gemm::launch_gemm(epi, prm, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int gemm_bf16(const void* a, const void* w, const float* bias, void* c, int M, int N, int K, int epilogue,
              void* stream) {
  return run_gemm(a, w, bias, c, M, N, K, epilogue, stream);
}

int attn_fwd_unfused(const void* q, const void* k, const void* v, float* o, float* lse, void* workspace,
                     unsigned long long workspace_bytes, int B, int H, int N, int d, int causal, float scale,
                     void* stream, int dtype) {
  return run_unfused(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, causal, scale, stream, dtype);
}

int attn_fwd_unfused_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N,
                             int d, int causal, float scale, void* stream, int dtype) {
  return run_unfused(q, k, v, o, lse, nullptr, 0, B, H, N, d, causal, scale, stream, dtype, true);
}

unsigned long long attn_unfused_workspace_bytes(int B, int H, int N) {
  if (!unfused_shape_ok(B, H, N, 64)) return 0;
  return unfused_ws_bytes(B, H, N);
}

int softmax_rows(const void* x, void* y, int rows, int cols, int dtype, void* stream) {
  return run_softmax(x, y, rows, cols, dtype, stream);
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
                  int N, int d, int causal, float scale, void* stream) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, ATTN_BF16, nullptr);
}

int attn_fwd_fp16(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
                  int N, int d, int causal, float scale, void* stream) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, ATTN_FP16, nullptr);
}

int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
             int N, int d, int causal, float scale, void* stream, int dtype) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, nullptr);
}

int attn_fwd_cfg(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
                 int N, int d, int causal, float scale, void* stream, int dtype,
                 const attn_launch_cfg* cfg) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, cfg);
}

int attn_resolve_cfg(int B, int H, int N, int d, int causal, int dtype, attn_launch_cfg* cfg) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (!cfg) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
  if (!shape_ok(B, H, N, d)) return ATTN_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (!cfg_valid(cfg, bh)) return ATTN_ERR_CONFIG;
  ttc::AttnParams prm{};
  prm.BH = (int)bh;
  prm.N = N;
  ttc::LaunchCfg c{cfg->n_dom, cfg->n_work, cfg->grp, cfg->prio, cfg->mode, cfg->tile};
  const hipError_t e = ttc::resolve_cfg(dtype == ATTN_BF16, d, causal == 1, prm, c);
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  cfg->n_dom = c.n_dom;
  cfg->n_work = c.n_work;
  cfg->grp = c.grp;
  cfg->prio = c.prio;
  cfg->mode = c.mode;
  cfg->tile = c.tile;
  return ATTN_OK;
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a pointer argument is NULL";
    case ATTN_ERR_SHAPE: return "B, H and N must be >= 1 and B*H*N*d within limits";
    case ATTN_ERR_UNSUPPORTED_D: return "head dimension d must be 64 or 128";
    case ATTN_ERR_ALIGN: return "every pointer must be 16-byte aligned";
    case ATTN_ERR_DTYPE: return "dtype must be ATTN_BF16 or ATTN_FP16";
    case ATTN_ERR_HIP: return "kernel launch failed (see attn_last_error)";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_CAUSAL: return "causal must be 0 or 1";
    case ATTN_ERR_ALIAS: return "o and lse must not overlap each other or q, k, v";
    case ATTN_ERR_CONFIG: return "launch configuration field out of range";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than the shape needs";
    case ATTN_ERR_SCRATCH: return "B*H*N*N*4 exceeds the built-in scratch (ATTN_UNFUSED_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_block_rows(int d) { return (d == 64 || d == 128) ? ttc::block_rows(ATTN_TILE_128) : 0; }

int attn_tile_info(int tile, int mode, int dtype, int d, int causal, attn_tile_resources* out) {
  if (!out) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
  attn_launch_cfg c{0, 0, 0, 0, mode, tile};
  if (!cfg_valid(&c, 8)) return ATTN_ERR_CONFIG;
  ttc::KernelInfo k{};
  const hipError_t e = ttc::kernel_info(dtype == ATTN_BF16, d, causal == 1, mode != ATTN_REF_RUNNING,
                                        tile == 0 ? ATTN_TILE_128 : tile, k);
  if (e != hipSuccess) {
    g_last_error = hipGetErrorString(e);
    return ATTN_ERR_HIP;
  }
  out->rows = k.rows;
  out->waves = k.waves;
  out->vgprs = k.vgprs;
  out->lds_bytes = k.lds_bytes;
  out->scratch_bytes = k.scratch_bytes;
  out->groups_per_cu = k.groups_per_cu;
  return ATTN_OK;
}

}  // extern "C"
