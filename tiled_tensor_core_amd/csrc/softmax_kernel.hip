// Row-wise softmax for gfx950 (CDNA4, wave64): y_ij = exp(x_ij - m_i) / sum_k
// exp(x_ik - m_i) over each row of a [rows, cols] matrix.
//
// Method: TileLang tutorial "Designing high-performance GPU kernels with a
// high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
// section on the fused GEMM epilogue and the row-wise softmax -- the row
// maximum and the row sum come from reductions over register fragments, and
// the normalisation stays in registers.
//
// The operation moves 2 * rows * cols * elem bytes and does a few VALU
// operations per element, so it is bound by HBM bandwidth; the design aims at
// keeping enough bytes in flight and reading every row once:
//   * rows of up to 16 KiB: one wave per row, rows dealt to the waves of a
//     grid sized to the chip (each wave loops over rows, rows apart by the
//     number of waves).  The row is read once into registers with 16-byte
//     buffer loads (64 lanes x 16 bytes per instruction, all issued before
//     the first use), kept packed, and walked three times: maximum, sum of
//     exponentials, normalised output (the exponential is recomputed rather
//     than kept, so a lane holds at most 64 VGPRs of row data and many waves
//     fit on a SIMD);
//   * rows of up to 256 KiB (fp32; 128 KiB for 16-bit types, whose unpacked
//     elements need twice the registers): one workgroup of 16 waves per row,
//     each wave holding its share in registers, so the row is still read
//     once; the row's maximum and sum combine across the waves through LDS;
//   * longer rows: one workgroup per row, read twice in 256 KiB segments --
//     an online pass keeps a running maximum and a sum rescaled when the
//     maximum moves, then a second pass writes the output;
//   * rows whose byte length is not a multiple of 16 (odd lengths of 16-bit
//     data) start at every alignment: one wave per row loads the aligned
//     interior with 16-byte loads and the head and tail (each under 16 bytes)
//     element by element, and keeps the row in registers like the first path;
//     such rows longer than 16 KiB take an element-wise path that re-reads
//     the row (mostly from cache);
//   * within a wave, results combine with xor shuffles;
//   * 16-byte output stores are non-temporal;
//   * exponentials are exp2 with log2(e) folded into one multiply-add.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "softmax_launch.h"

namespace ttc_sm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define SM_INLINE __device__ __attribute__((always_inline)) inline

constexpr float kLog2e = 1.4426950408889634074f;
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kMaxChunks = 16;       // 16-byte pieces per lane: rows of up to 16 KiB in registers
// Output stores carry the non-temporal cache policy (bit 1, "nt" on gfx950):
// the output is written once and never read back here, and streaming it
// past the caches keeps them for the input (a 256 MiB fp32 softmax runs
// about a fifth faster; inputs that fit the caches are unaffected).
constexpr int kStoreNT = 2;

// Element type T: 0 fp32, 1 bf16, 2 fp16.
template <int T>
struct Elem;
template <>
struct Elem<0> {
  static constexpr int kBytes = 4, kPerWord = 1;
  SM_INLINE static float get(uint32_t w, int k) { (void)k; return __builtin_bit_cast(float, w); }
  SM_INLINE static uint32_t put(float a, float b) { (void)b; return __builtin_bit_cast(uint32_t, a); }
};
template <>
struct Elem<1> {
  static constexpr int kBytes = 2, kPerWord = 2;
  SM_INLINE static float get(uint32_t w, int k) { return __builtin_bit_cast(float, k ? (w & 0xffff0000u) : (w << 16)); }
  SM_INLINE static uint32_t put(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
};
template <>
struct Elem<2> {
  static constexpr int kBytes = 2, kPerWord = 2;
  SM_INLINE static float get(uint32_t w, int k) {
    return (float)__builtin_bit_cast(f16x2, w)[k];
  }
  SM_INLINE static uint32_t put(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
};

SM_INLINE float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = __builtin_elementwise_maximum(v, __shfl_xor(v, m, 64));
  return v;
}
SM_INLINE float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
SM_INLINE float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

SM_INLINE __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

// Every exponential is ex2(fma(x, log2e, -c)) with the offset c = m * log2e
// rounded once to fp32, and every partial sum is kept against such a rounded
// offset: s = sum ex2(x * log2e - c(m)).  Moving a sum to a larger maximum
// multiplies it by ex2(c(m) - c(mn)), the difference of the two rounded
// offsets, so the numerators written at the end (against c(M)) and the
// denominator carry the same offset and its rounding cancels.  (Rescaling by
// ex2((m - mn) * log2e) instead leaves the rounding of c(M) in the numerators
// only: a relative error of up to ulp(M * log2e), 1e-3 for |M| ~ 1e4.)
SM_INLINE float offset(float m) {
#pragma clang fp contract(off)
  return m * kLog2e;
}
SM_INLINE float shift(float cm, float cn) {
#pragma clang fp contract(off)
  return ex2(cm - cn);
}

// Natural log-sum-exp of a row from its offset c(m) and its sum s against
// that offset: sum_j e^x_j = 2^(c(m)) * s.
SM_INLINE float row_lse(float cm, float s) {
  return (cm + __builtin_amdgcn_logf(s)) * 0.69314718055994530942f;
}

// Running (maximum, sum) of one lane, the sum taken against offset(m): merge
// a block maximum mb and block sum sb taken against offset(mb).  A side with
// no element yet has m = -inf, s = 0.
SM_INLINE void merge(float& m, float& s, float mb, float sb) {
  const float mn = __builtin_elementwise_maximum(m, mb);
  const float cn = offset(mn);
  const float fa = (m == -INFINITY) ? 0.0f : shift(offset(m), cn);
  const float fb = (mb == -INFINITY) ? 0.0f : shift(offset(mb), cn);
  s = s * fa + sb * fb;
  m = mn;
}

// Rows of at most NCH * 1 KiB whose byte length is a multiple of 16.
template <int T, int NCH>
__global__ void __launch_bounds__(kWaves * 64) softmax_reg(const uint8_t* x, uint8_t* y, int rows, int row_bytes, float* lse) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  for (int r = blockIdx.x * kWaves + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const size_t roff = (size_t)r * (size_t)row_bytes;
    const __amdgpu_buffer_rsrc_t xs = rsrc(x + roff, (uint32_t)row_bytes);
    u32x4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c] = __builtin_amdgcn_raw_buffer_load_b128(xs, (c * 64 + lane) * 16, 0, 0);
    // a 16-byte piece is wholly inside the row or wholly past it
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if ((c * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) m = __builtin_elementwise_maximum(m, E::get(v[c][w], k));
    }
    m = wave_max(m);
    const float mc = offset(m);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if ((c * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) s += ex2(__builtin_fmaf(E::get(v[c][w], k), kLog2e, -mc));
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
    if (lse && lane == 0) lse[r] = row_lse(mc, s);
    const __amdgpu_buffer_rsrc_t ys = rsrc(y + roff, (uint32_t)row_bytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = ex2(__builtin_fmaf(E::get(v[c][w], 0), kLog2e, -mc)) * inv;
        const float b = E::kPerWord == 2 ? ex2(__builtin_fmaf(E::get(v[c][w], 1), kLog2e, -mc)) * inv : 0.0f;
        o[w] = E::put(a, b);
      }
      // pieces past the row fall outside the buffer and are dropped
      __builtin_amdgcn_raw_buffer_store_b128(o, ys, (c * 64 + lane) * 16, 0, kStoreNT);
    }
  }
}

// Maximum and sum over the kBlockWaves waves of a workgroup: each wave's
// value goes through LDS slot red[w]; the barrier also orders the slot's
// reuse, since a wave reads the maximum slots before it writes a sum slot
// and the next row's maximum slots are written only after the sum barrier.
constexpr int kBlockWaves = 16;      // waves per workgroup on the row-per-workgroup paths

SM_INLINE float block_reduce(float v, float* red, bool is_max) {
  const int w = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < kBlockWaves; ++i) a = is_max ? __builtin_elementwise_maximum(a, red[i]) : a + red[i];
  return a;
}

// Pieces per wave on the row-per-workgroup register path: a workgroup of 16
// waves leaves a wave 128 VGPRs, which hold 16 KiB of fp32 row but only
// 8 KiB of 16-bit row once its elements are unpacked to fp32.
template <int T>
constexpr int kBlkChunks = T == 0 ? kMaxChunks : kMaxChunks / 2;

// Rows of at most kBlockWaves * NCH KiB (byte length a multiple of 16), one
// row per workgroup: wave w of the workgroup holds the 1 KiB pieces
// c * kBlockWaves + w (c < NCH) of the row in registers, so the row is read
// once; the row's maximum and sum combine across the waves through LDS.
template <int T, int NCH>
__global__ void __launch_bounds__(kBlockWaves * 64) softmax_blk(const uint8_t* x, uint8_t* y, int rows, int row_bytes, float* lse) {
  using E = Elem<T>;
  __shared__ float red_max[kBlockWaves], red_sum[kBlockWaves];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const size_t roff = (size_t)r * (size_t)row_bytes;
    const __amdgpu_buffer_rsrc_t xs = rsrc(x + roff, (uint32_t)row_bytes);
    u32x4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      v[c] = __builtin_amdgcn_raw_buffer_load_b128(xs, ((c * kBlockWaves + wv) * 64 + lane) * 16, 0, 0);
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (((c * kBlockWaves + wv) * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) m = __builtin_elementwise_maximum(m, E::get(v[c][w], k));
    }
    const float mc = offset(block_reduce(m, red_max, true));
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (((c * kBlockWaves + wv) * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) s += ex2(__builtin_fmaf(E::get(v[c][w], k), kLog2e, -mc));
    }
    const float tot = block_reduce(s, red_sum, false);
    const float inv = 1.0f / tot;
    if (lse && threadIdx.x == 0) lse[r] = row_lse(mc, tot);
    const __amdgpu_buffer_rsrc_t ys = rsrc(y + roff, (uint32_t)row_bytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = ex2(__builtin_fmaf(E::get(v[c][w], 0), kLog2e, -mc)) * inv;
        const float b = E::kPerWord == 2 ? ex2(__builtin_fmaf(E::get(v[c][w], 1), kLog2e, -mc)) * inv : 0.0f;
        o[w] = E::put(a, b);
      }
      __builtin_amdgcn_raw_buffer_store_b128(o, ys, ((c * kBlockWaves + wv) * 64 + lane) * 16, 0, kStoreNT);
    }
  }
}

// Rows longer than a workgroup's registers hold, byte length a multiple of
// 16: one row per workgroup, read twice in segments of kBlockWaves *
// kMaxChunks KiB.  The first pass keeps a running (maximum, sum) per lane;
// the lanes' pairs combine across the workgroup; the second pass writes.
template <int T>
__global__ void __launch_bounds__(kBlockWaves * 64) softmax_seg(const uint8_t* x, uint8_t* y, int rows, int row_bytes, float* lse) {
  using E = Elem<T>;
  constexpr int SEG = kBlockWaves * kMaxChunks * 1024;
  __shared__ float red_max[kBlockWaves], red_sum[kBlockWaves];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const size_t roff = (size_t)r * (size_t)row_bytes;
    float m = -INFINITY, s = 0.0f;
    for (int seg = 0; seg < row_bytes; seg += SEG) {
      // one resource per segment, so the range check sees the whole offset
      const __amdgpu_buffer_rsrc_t xs = rsrc(x + roff + seg, (uint32_t)(row_bytes - seg));
      u32x4 v[kMaxChunks];
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        v[c] = __builtin_amdgcn_raw_buffer_load_b128(xs, ((c * kBlockWaves + wv) * 64 + lane) * 16, 0, 0);
      float mb = -INFINITY;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        if (seg + ((c * kBlockWaves + wv) * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int k = 0; k < E::kPerWord; ++k) mb = __builtin_elementwise_maximum(mb, E::get(v[c][w], k));
      }
      float sb = 0.0f;
      if (mb != -INFINITY) {
        const float mc = offset(mb);
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          if (seg + ((c * kBlockWaves + wv) * 64 + lane) * 16 >= row_bytes) continue;
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int k = 0; k < E::kPerWord; ++k) sb += ex2(__builtin_fmaf(E::get(v[c][w], k), kLog2e, -mc));
        }
      }
      merge(m, s, mb, sb);
    }
    const float M = block_reduce(m, red_max, true);
    const float mc = offset(M);
    const float tot = block_reduce((m == -INFINITY) ? 0.0f : s * shift(offset(m), mc), red_sum, false);
    const float inv = 1.0f / tot;
    if (lse && threadIdx.x == 0) lse[r] = row_lse(mc, tot);
    for (int seg = 0; seg < row_bytes; seg += SEG) {
      const __amdgpu_buffer_rsrc_t xs = rsrc(x + roff + seg, (uint32_t)(row_bytes - seg));
      const __amdgpu_buffer_rsrc_t ys = rsrc(y + roff + seg, (uint32_t)(row_bytes - seg));
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        const int off = ((c * kBlockWaves + wv) * 64 + lane) * 16;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0);
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a = ex2(__builtin_fmaf(E::get(v[w], 0), kLog2e, -mc)) * inv;
          const float b = E::kPerWord == 2 ? ex2(__builtin_fmaf(E::get(v[w], 1), kLog2e, -mc)) * inv : 0.0f;
          o[w] = E::put(a, b);
        }
        __builtin_amdgcn_raw_buffer_store_b128(o, ys, off, 0, kStoreNT);
      }
    }
  }
}

// Rows of at most NCH KiB whose byte length is not a multiple of 16 (odd
// lengths of 16-bit data, or fp32 rows of a length not divisible by 4), so
// rows start at every alignment: one wave per row.  The row's 16-byte
// aligned interior is read with 16-byte buffer loads (64 lanes x 16 bytes per
// instruction, all issued before the first use), the head before it and the
// tail after it (each under 16 bytes) element by element by lanes 0-7 and
// 8-15; everything stays in registers for the three passes (maximum, sum,
// output), and the interior is written with 16-byte stores.
template <int T, int NCH>
__global__ void __launch_bounds__(kWaves * 64) softmax_odd(const uint8_t* x, uint8_t* y, int rows, int cols,
                                                         float* lse) {
  using E = Elem<T>;
  constexpr int EB = E::kBytes;
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  const int row_bytes = cols * EB;
  auto load1 = [&](const uint8_t* p) -> float {
    if (EB == 4) return *reinterpret_cast<const float*>(p);
    return E::get(*reinterpret_cast<const uint16_t*>(p), 0);
  };
  auto store1 = [&](uint8_t* p, float v) {
    if (EB == 4)
      *reinterpret_cast<float*>(p) = v;
    else
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)(E::put(v, 0.0f) & 0xffffu);
  };
  for (int r = blockIdx.x * kWaves + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const size_t roff = (size_t)r * (size_t)row_bytes;
    const int hb = min((int)((16 - (roff & 15)) & 15), row_bytes);   // head bytes, up to the first 16-byte boundary
    const int ib = ((row_bytes - hb) >> 4) << 4;                      // aligned interior bytes
    const int tb = row_bytes - hb - ib;                               // tail bytes (< 16)
    const __amdgpu_buffer_rsrc_t xs = rsrc(x + roff + hb, (uint32_t)ib);
    u32x4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c] = __builtin_amdgcn_raw_buffer_load_b128(xs, (c * 64 + lane) * 16, 0, 0);
    // lanes 0-7: head element `lane`; lanes 8-15: tail element `lane - 8`; -inf elsewhere (weight 0)
    const bool in_head = lane * EB < hb;
    const bool in_tail = lane >= 8 && (lane - 8) * EB < tb;
    const size_t eoff = in_head ? roff + (size_t)(lane * EB) : roff + (size_t)(hb + ib + (lane - 8) * EB);
    const float hv = (in_head || in_tail) ? load1(x + eoff) : -INFINITY;
    float m = hv;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if ((c * 64 + lane) * 16 >= ib) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) m = __builtin_elementwise_maximum(m, E::get(v[c][w], k));
    }
    m = wave_max(m);
    const float mc = offset(m);
    float s = (in_head || in_tail) ? ex2(__builtin_fmaf(hv, kLog2e, -mc)) : 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if ((c * 64 + lane) * 16 >= ib) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < E::kPerWord; ++k) s += ex2(__builtin_fmaf(E::get(v[c][w], k), kLog2e, -mc));
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
    if (lse && lane == 0) lse[r] = row_lse(mc, s);
    const __amdgpu_buffer_rsrc_t ys = rsrc(y + roff + hb, (uint32_t)ib);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = ex2(__builtin_fmaf(E::get(v[c][w], 0), kLog2e, -mc)) * inv;
        const float b = E::kPerWord == 2 ? ex2(__builtin_fmaf(E::get(v[c][w], 1), kLog2e, -mc)) * inv : 0.0f;
        o[w] = E::put(a, b);
      }
      // pieces past the interior fall outside the buffer and are dropped
      __builtin_amdgcn_raw_buffer_store_b128(o, ys, (c * 64 + lane) * 16, 0, kStoreNT);
    }
    if (in_head || in_tail) store1(y + eoff, ex2(__builtin_fmaf(hv, kLog2e, -mc)) * inv);
  }
}

// Any row: element-wise loads (lane j takes elements j, j + 64, ...) and the
// register path's three passes (maximum, sum, output), the second and third
// reading the row again.  Used when a row's byte length is not a multiple of
// 16, so 16-byte loads do not apply.
template <int T>
__global__ void __launch_bounds__(kWaves * 64) softmax_elem(const uint8_t* x, uint8_t* y, int rows, int cols, float* lse) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  for (int r = blockIdx.x * kWaves + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const size_t rbase = (size_t)r * (size_t)cols;
    auto load = [&](int j) -> float {
      if (E::kBytes == 4) return reinterpret_cast<const float*>(x)[rbase + j];
      const uint32_t h = reinterpret_cast<const uint16_t*>(x)[rbase + j];
      return E::get(h, 0);
    };
    float m = -INFINITY;
    for (int j = lane; j < cols; j += 64) m = __builtin_elementwise_maximum(m, load(j));
    const float mc = offset(wave_max(m));
    float s = 0.0f;
    for (int j = lane; j < cols; j += 64) s += ex2(__builtin_fmaf(load(j), kLog2e, -mc));
    const float tot = wave_sum(s);
    const float inv = 1.0f / tot;
    if (lse && lane == 0) lse[r] = row_lse(mc, tot);
    for (int j = lane; j < cols; j += 64) {
      const float p = ex2(__builtin_fmaf(load(j), kLog2e, -mc)) * inv;
      // plain stores: the caches merge the lanes' partial lines before they
      // reach HBM (non-temporal 2-byte stores write about 1.6x the bytes)
      if (E::kBytes == 4) {
        reinterpret_cast<float*>(y)[rbase + j] = p;
      } else {
        reinterpret_cast<uint16_t*>(y)[rbase + j] = (uint16_t)(E::put(p, 0.0f) & 0xffffu);
      }
    }
  }
}

// Compute units of the current device (the runtime caches the attribute).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    return n;
  return 256;
}

// Wave-per-row paths: as many workgroups of kWaves waves as the device keeps
// busy (a few per CU), or fewer for few rows.
static int grid_for(int rows) {
  const long long want = ((long long)rows + kWaves - 1) / kWaves;
  const long long cap = (long long)cu_count() * 8;
  return (int)(want < cap ? want : cap);
}

// Row-per-workgroup paths: one workgroup per row, at most two per CU at once.
static int grid_blocks(int rows) {
  const long long cap = (long long)cu_count() * 2;
  return (int)(rows < cap ? rows : cap);
}

template <int T>
static hipError_t launch_t(const void* x, void* y, int rows, int cols, float* lse, hipStream_t stream) {
  const long long row_bytes = (long long)cols * Elem<T>::kBytes;
  const dim3 block(kWaves * 64);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* yb = static_cast<uint8_t*>(y);
  if (row_bytes % 16 != 0) {
    const int op = (int)((row_bytes + 1023) / 1024);   // 1 KiB pieces of the interior, at most
    const dim3 grid(grid_for(rows));
    if (op <= 1)
      hipLaunchKernelGGL((softmax_odd<T, 1>), grid, block, 0, stream, xb, yb, rows, cols, lse);
    else if (op <= 2)
      hipLaunchKernelGGL((softmax_odd<T, 2>), grid, block, 0, stream, xb, yb, rows, cols, lse);
    else if (op <= 4)
      hipLaunchKernelGGL((softmax_odd<T, 4>), grid, block, 0, stream, xb, yb, rows, cols, lse);
    else if (op <= 8)
      hipLaunchKernelGGL((softmax_odd<T, 8>), grid, block, 0, stream, xb, yb, rows, cols, lse);
    else if (op <= kMaxChunks)
      hipLaunchKernelGGL((softmax_odd<T, kMaxChunks>), grid, block, 0, stream, xb, yb, rows, cols, lse);
    else
      hipLaunchKernelGGL(softmax_elem<T>, grid, block, 0, stream, xb, yb, rows, cols, lse);
    return hipGetLastError();
  }
  const int rb = (int)row_bytes;
  const int pieces = (rb + 1023) / 1024;   // 1 KiB per wave-wide 16-byte load
  if (pieces <= kMaxChunks) {
    const dim3 grid(grid_for(rows));
    if (pieces <= 1)
      hipLaunchKernelGGL((softmax_reg<T, 1>), grid, block, 0, stream, xb, yb, rows, rb, lse);
    else if (pieces <= 2)
      hipLaunchKernelGGL((softmax_reg<T, 2>), grid, block, 0, stream, xb, yb, rows, rb, lse);
    else if (pieces <= 4)
      hipLaunchKernelGGL((softmax_reg<T, 4>), grid, block, 0, stream, xb, yb, rows, rb, lse);
    else if (pieces <= 8)
      hipLaunchKernelGGL((softmax_reg<T, 8>), grid, block, 0, stream, xb, yb, rows, rb, lse);
    else
      hipLaunchKernelGGL((softmax_reg<T, kMaxChunks>), grid, block, 0, stream, xb, yb, rows, rb, lse);
    return hipGetLastError();
  }
  // one row per workgroup of kBlockWaves waves
  const dim3 bblock(kBlockWaves * 64);
  const dim3 bgrid(grid_blocks(rows));
  const int per_wave = (pieces + kBlockWaves - 1) / kBlockWaves;
  if (per_wave <= 2)
    hipLaunchKernelGGL((softmax_blk<T, 2>), bgrid, bblock, 0, stream, xb, yb, rows, rb, lse);
  else if (per_wave <= 4)
    hipLaunchKernelGGL((softmax_blk<T, 4>), bgrid, bblock, 0, stream, xb, yb, rows, rb, lse);
  else if (per_wave <= 8)
    hipLaunchKernelGGL((softmax_blk<T, 8>), bgrid, bblock, 0, stream, xb, yb, rows, rb, lse);
  else if (per_wave <= kBlkChunks<T>)
    hipLaunchKernelGGL((softmax_blk<T, kBlkChunks<T>>), bgrid, bblock, 0, stream, xb, yb, rows, rb, lse);
  else
    hipLaunchKernelGGL(softmax_seg<T>, bgrid, bblock, 0, stream, xb, yb, rows, rb, lse);
  return hipGetLastError();
}

hipError_t launch_softmax(int dtype, const void* x, void* y, int rows, int cols, float* lse, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_t<0>(x, y, rows, cols, lse, stream);
    case 1: return launch_t<1>(x, y, rows, cols, lse, stream);
    default: return launch_t<2>(x, y, rows, cols, lse, stream);
  }
}

}  // namespace ttc_sm
