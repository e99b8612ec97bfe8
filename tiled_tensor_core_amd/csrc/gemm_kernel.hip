// Tiled bf16 GEMM with a fused bias + GELU epilogue for gfx950 (CDNA4, wave64):
//
//     C[m, n] = epilogue( sum_k A[m, k] * W[n, k]  (+ bias[n]) )
//
// Method: TileLang tutorial "Designing high-performance GPU kernels with a
// high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
// sections on the tiled tensor-core matrix multiplication (tiles staged from
// global memory through shared memory into register fragments for the
// matrix cores) and on the fused GEMM epilogue (bias and GELU applied to the
// accumulator in registers before the one write of the output).
//
// gfx950 design:
//   * a workgroup of 4 waves computes a 256 x 256 tile of C; each wave owns
//     a 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
//     accumulators (256 fp32 per lane, in the accumulation registers).
//   * K advances 64 at a time.  A [256 x 64] and W [256 x 64] slices go
//     from HBM straight into LDS with buffer_load_dwordx4 ... lds (16 bytes
//     per lane, 1 KiB per wave instruction), double-buffered: the loads of
//     slice j+1 are issued in the last k16 step of slice j-1 and land while
//     the MFMAs consume slice j; that last step also reads slice j's first
//     fragments, so no slice starts by waiting for LDS.
//     The two buffers are distinct LDS objects and the loop is unrolled by
//     two, so the compiler can tell the DMA target from the buffer being
//     read.
//   * an LDS row holds 64 k values (8 chunks of 16 bytes); the chunk index
//     is XOR-swizzled with (row >> 1) & 7: the 16 lanes of a phase of a
//     fragment read (rows r .. r+15 at one chunk, 256 bytes of LDS banks)
//     then hit 16 different 16-byte bank groups.
//   * both operands are K-contiguous (A [M, K], W [N, K]), so both
//     fragments are plain 16-byte LDS reads.  W is the MFMA's first operand
//     and A the second: the accumulator block is then C^T, and each lane
//     holds one row m of C with four runs of 4 consecutive columns n.
//   * the bias is the accumulators' starting value, so the matrix cores add
//     the products to it; the epilogue in registers applies GELU(z) =
//     z * erfc(-z / sqrt 2) / 2 (erfc from Abramowitz and Stegun 7.1.26)
//     and rounds to bf16; then each wave stages its 128 x 128 bf16 quarter
//     in LDS (rows of 256 bytes, 16-byte chunks XOR-swizzled with row & 15,
//     the 8-byte halves of a chunk swapped in rows with bit 4 set) and
//     writes C in whole 16-byte pieces, 4 rows of 256 bytes per wave
//     instruction.
//   * tile order: workgroup b runs on XCD b % 8; the tiles are numbered in
//     groups of 4 tile-rows (column by column within a group), and XCD x
//     takes a contiguous range of those numbers, so the 32 tiles an XCD
//     runs at once share 4 row slices of A and 8 of W in its L2.
//   * ragged edges: rows of A or W past M or N read as zero (the buffer
//     range of the tile's resource); k chunks past K are sent out of range
//     and read as zero; stores past M or N are dropped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_launch.h"

namespace ttc_gemm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

#define G_INLINE __device__ __attribute__((always_inline)) inline

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWaves = 4;
constexpr int kRowBytes = kBK * 2;                    // 128 bytes of k per LDS row
constexpr int kSliceBytes = kBM * kRowBytes;          // 32 KiB per operand slice
constexpr int kLoadsPerWave = kSliceBytes / (kWaves * 1024);   // 8 per operand
constexpr int kGroupRows = 4;                         // tile-rows per group in the tile order
constexpr uint32_t kOut = 0x80000000u;                // a buffer offset past any range

static_assert(kSliceBytes % (kWaves * 1024) == 0, "a slice must split evenly over the waves");

G_INLINE __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

G_INLINE f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

G_INLINE u32x4 lds_read16(const lds_u8* p) { return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p); }

// erfc by Abramowitz and Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erfc(x) ~ t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) exp(-x^2),
// t = 1 / (1 + p x), for x >= 0 (absolute error below 1.5e-7), and
// erfc(-x) = 2 - erfc(x).  Over z in [-12, 12] the GELU built on it stays
// within 4.3e-7 of the exact one in fp32 (at most 1.7e-4 relative where
// |GELU| > 1e-3), far below the bf16 rounding of the output, at a fifth of
// the instructions of the library erfcf.
G_INLINE float erfc_as(float x) {
  const float ax = __builtin_fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = poly * __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return x >= 0.0f ? e : 2.0f - e;
}
// GELU(z) = z * Phi(z), Phi(z) = erfc(-z / sqrt(2)) / 2 (no cancellation for
// negative z).
G_INLINE float gelu(float z) { return 0.5f * z * erfc_as(-0.70710678118654752f * z); }

// The accumulator already holds the bias (when there is one); only the
// activation is left.
template <int EPI>
G_INLINE float activation(float z) {
  if constexpr (EPI == 2) {
    return gelu(z);
  } else {
    return z;
  }
}

template <int EPI>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[kSliceBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds0[kSliceBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds1[kSliceBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds1[kSliceBytes];
  lds_u8* const A0 = (lds_u8*)a_lds0;
  lds_u8* const W0 = (lds_u8*)w_lds0;
  lds_u8* const A1 = (lds_u8*)a_lds1;
  lds_u8* const W1 = (lds_u8*)w_lds1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;             // this wave's quarter of the tile

  // ---- tile of this workgroup ---------------------------------------------
  const int nt = (int)gridDim.x, b = (int)blockIdx.x;
  const int x = b & 7, i = b >> 3, q = nt >> 3, r = nt & 7;
  const int t = x * q + min(x, r) + i;                 // XCD x: tiles [x*q + min(x, r), +q + (x < r))
  const int span = kGroupRows * p.tiles_n;
  const int first_m = (t / span) * kGroupRows;
  const int gm = min(kGroupRows, p.tiles_m - first_m);
  const int u = t - (t / span) * span;
  const int tm = first_m + u % gm, tn = u / gm;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- operand loads: HBM -> LDS ----------------------------------------------
  // Load t of a wave fills LDS bytes [(wave*8 + t) KiB, +1 KiB): chunk index
  // idx = (wave*8 + t)*64 + lane, row idx / 8, swizzled chunk idx % 8, which
  // holds logical chunk (idx % 8) ^ ((row >> 1) & 7): k = 8 * that chunk.
  const uint32_t a_rows = (uint32_t)min(kBM, M - m0), w_rows = (uint32_t)min(kBN, N - n0);
  const __amdgpu_buffer_rsrc_t ars = rsrc(p.a + (size_t)m0 * K, a_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wrs = rsrc(p.w + (size_t)n0 * K, w_rows * (uint32_t)K * 2u);
  int ld_row[kLoadsPerWave], ld_k[kLoadsPerWave];
#pragma unroll
  for (int s = 0; s < kLoadsPerWave; ++s) {
    const int idx = (wave * kLoadsPerWave + s) * 64 + lane;
    const int row = idx >> 3;
    ld_row[s] = row;
    ld_k[s] = 8 * ((idx & 7) ^ ((row >> 1) & 7));
  }
  auto load_slice = [&](lds_u8* abuf, lds_u8* wbuf, int k0) {
#pragma unroll
    for (int s = 0; s < kLoadsPerWave; ++s) {
      const int k = k0 + ld_k[s];
      const uint32_t off = k < K ? (uint32_t)(ld_row[s] * K + k) * 2u : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(abuf + (wave * kLoadsPerWave + s) * 1024), 16, off,
                                               0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < kLoadsPerWave; ++s) {
      const int k = k0 + ld_k[s];
      const uint32_t off = k < K ? (uint32_t)(ld_row[s] * K + k) * 2u : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void*)(wbuf + (wave * kLoadsPerWave + s) * 1024), 16, off,
                                               0, 0, 0);
    }
  };

  // ---- fragment reads: lane l reads row l % 32 of a 32-row block, k chunk
  // 2*kk + l / 32 of the slice, at its swizzled place.
  int rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) rd[kk] = (lane & 31) * kRowBytes + (((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4);
  const int a_base = wm * 128 * kRowBytes, w_base = wn * 128 * kRowBytes;

  // Accumulators start at the bias (register 4g + jj of a lane in column
  // block nb is column nb*32 + 8g + 4*(lane / 32) + jj, for every row block),
  // so the matrix cores add the products on top and no epilogue add is left.
  f32x16 acc[4][4];
  {
    const int h4 = 4 * (lane >> 5);
    const __amdgpu_buffer_rsrc_t brs = rsrc(p.bias, EPI != 0 ? (uint32_t)N * 4u : 0u);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x16 bv = {};
      if constexpr (EPI != 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + nb * 32 + 8 * g + h4;
          const f32x4 b4 = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, n < N ? (uint32_t)n * 4u : kOut, 0, 0));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) bv[4 * g + jj] = b4[jj];
        }
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = bv;
    }
  }

  // Fragment reads run one k16 step ahead of the MFMAs that use them, and
  // scheduling group barriers interleave them with the MFMAs, one read
  // between every two MFMAs.  LDS is the busiest unit here -- the loads
  // write 64 KiB and the fragment reads read 128 KiB per slice per compute
  // unit -- and a burst of reads from all four waves queued behind the load
  // traffic stalled the matrix cores; spread out, the same work ran 3-8 %
  // faster.  A scheduling barrier closes each step, so no read moves up
  // into an earlier step.
  auto read_frags = [&](const lds_u8* abuf, const lds_u8* wbuf, int kk, u32x4 (&af)[4], u32x4 (&wf)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[mb] = lds_read16(abuf + a_base + mb * 32 * kRowBytes + rd[kk]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) wf[nb] = lds_read16(wbuf + w_base + nb * 32 * kRowBytes + rd[kk]);
  };
  // The first k16 step of a slice reads its fragments during the last step
  // of the slice before: that step waits for the next slice's loads and
  // holds the barrier after its first four MFMAs, then reads the next
  // slice's first fragments and issues the loads of the slice after it
  // (into the buffer just read) between its remaining MFMAs.  So no slice
  // starts by waiting for LDS.  Two fragment register sets alternate:
  // A (af0/wf0) for steps 0 and 2, B for steps 1 and 3.
  u32x4 af0[4], wf0[4];
  auto compute = [&](const lds_u8* abuf, const lds_u8* wbuf, const lds_u8* nabuf, const lds_u8* nwbuf,
                     lds_u8* dabuf, lds_u8* dwbuf, int dk0) {
    u32x4 af1[4], wf1[4];
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      if (kk & 1)
        read_frags(abuf, wbuf, kk + 1, af0, wf0);
      else
        read_frags(abuf, wbuf, kk + 1, af1, wf1);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = (kk & 1) ? mfma(wf1[nb], af1[mb], acc[mb][nb]) : mfma(wf0[nb], af0[mb], acc[mb][nb]);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // step 3
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[0][nb] = mfma(wf1[nb], af1[0], acc[0][nb]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(nabuf, nwbuf, 0, af0, wf0);
    load_slice(dabuf, dwbuf, dk0);
#pragma unroll
    for (int mb = 1; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma(wf1[nb], af1[mb], acc[mb][nb]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      if (g < 6) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop: two slices per iteration, one per buffer --------------------
  // The slice count is rounded up to even (a slice past K reads as zeros),
  // so the loop has one exit and the accumulators one loop-carried copy.
  // The last two slices issue loads past K, which only write zeros into
  // LDS; the barrier after the loop waits for them.
  const int nk = ((K + kBK - 1) / kBK + 1) & ~1;
  load_slice(A0, W0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  load_slice(A1, W1, kBK);
  read_frags(A0, W0, 0, af0, wf0);
  for (int j = 0; j < nk; j += 2) {
    compute(A0, W0, A1, W1, A0, W0, (j + 2) * kBK);   // slice j; reads slice j+1, loads slice j+2
    compute(A1, W1, A0, W0, A1, W1, (j + 3) * kBK);   // slice j+1; reads slice j+2, loads slice j+3
  }
  // every wave is done reading the slices: LDS is free for the output.  The
  // scheduling barriers keep the accumulator reads of the epilogue below
  // it (hoisted above, all 256 values would sit in VGPRs at once).
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue -------------------------------------------------------------
  // Lane l holds, for block (mb, nb), row m = mb*32 + l % 32 of the wave's
  // quarter and columns nb*32 + 8g + 4*(l / 32) + jj for register 4g + jj.
  // Each wave stages its quarter in one 32 KiB LDS object.
  lds_u8* const stage = wave == 0 ? A0 : wave == 1 ? W0 : wave == 2 ? A1 : W1;
  const int h = lane >> 5, ml = lane & 31;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = mb * 32 + ml;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v0 = activation<EPI>(acc[mb][nb][4 * g + 0]);
        const float v1 = activation<EPI>(acc[mb][nb][4 * g + 1]);
        const float v2 = activation<EPI>(acc[mb][nb][4 * g + 2]);
        const float v3 = activation<EPI>(acc[mb][nb][4 * g + 3]);
        u32x2 pk;
        pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v0, v1}, bf16x2));
        pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v2, v3}, bf16x2));
        const int chunk = nb * 4 + g;                  // 16-byte chunk of the 256-byte row
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * (h ^ ((row >> 4) & 1))) = pk;
      }
      __builtin_amdgcn_sched_barrier(0);   // one block at a time: no hoisting of every block's values
    }
  }
  // each wave reads back only what it wrote
  const uint32_t c_rows = (uint32_t)min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t crs = rsrc(p.c + (size_t)m0 * N, c_rows * (uint32_t)N * 2u);
  const int c = lane & 15;
  const int n = n0 + wn * 128 + c * 8;
#pragma unroll
  for (int it = 0; it < 32; ++it) {
    const int row = it * 4 + (lane >> 4);
    u32x4 v = lds_read16(stage + row * 256 + ((c ^ (row & 15)) << 4));
    if ((it >> 2) & 1) v = (u32x4){v[2], v[3], v[0], v[1]};   // rows with bit 4 set hold their halves swapped
    const uint32_t off = n < N ? ((uint32_t)(wm * 128 + row) * (uint32_t)N + (uint32_t)n) * 2u : kOut;
    __builtin_amdgcn_raw_buffer_store_b128(v, crs, off, 0, 0);
  }
}

hipError_t launch_gemm(int epi, const GemmParams& prm, hipStream_t stream) {
  GemmParams p = prm;
  p.tiles_m = (p.M + kBM - 1) / kBM;
  p.tiles_n = (p.N + kBN - 1) / kBN;
  const long long tiles = (long long)p.tiles_m * p.tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)tiles), block(kWaves * 64);
  switch (epi) {
    case 0: hipLaunchKernelGGL(gemm_kernel<0>, grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(gemm_kernel<2>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace ttc_gemm



