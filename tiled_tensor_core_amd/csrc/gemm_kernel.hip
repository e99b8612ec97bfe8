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
// gfx950 design.  Three kernels share the tile layout, operand order,
// fragment reads, swizzle, accumulation order and epilogue, so C is the same
// bit for bit whichever runs:
//   * gemm_kernel4, for problems of at least 256 tiles of 256 x 256 with K a
//     multiple of 64: one workgroup of 4 waves per CU, one wave per SIMD,
//     128 x 128 of the tile per wave (8 x 8 MFMA blocks, 256 accumulators a
//     lane in the accumulation registers).  The operand slices reach LDS
//     straight from memory (buffer_load ... lds), so a k32 step issues only
//     its 64 MFMAs, 16 fragment reads for the next step and, every other
//     step, 16 loads; half the LDS instructions per MFMA of the 8-wave form.
//   * gemm_kernel (described below) for the other large problems;
//   * gemm_kernel_small for up to 128 tiles.
// The 8-wave kernel:
//   * a workgroup of 8 waves (two per SIMD) computes a 256 x 256 tile of C;
//     each wave owns 64 x 128 of it as 4 x 8 blocks of
//     v_mfma_f32_16x16x32_bf16 accumulators (128 fp32 per lane).  While one
//     wave of a SIMD issues its loads, LDS writes and fragment reads, the
//     other keeps the matrix core busy.  The 16x16x32 form does the same
//     work per cycle as 32x32x16 but draws less power on random data, so the
//     power-limited chip keeps a higher clock (measured: +14 % throughput for
//     back-to-back MFMAs on random bf16).
//   * K advances 64 at a time: A [256 x 64] and W [256 x 64] slices, double-
//     buffered in LDS.  Each wave moves 8 pieces of 1 KiB per slice
//     (16 bytes per lane) global -> VGPRs -> LDS: it loads the pieces of
//     slice j+2 during slice j and writes them to LDS during slice j+1, one
//     piece at a time between the MFMAs (A pieces in the slice's first k32
//     step, W pieces in the second), so every load keeps a slice of lead.
//     Loads straight into LDS (buffer_load ... lds) measured slower here.
//   * a k32 step is 8 groups of 4 MFMAs (group nb: W fragment nb against the
//     wave's 4 A fragments).  W fragments are read two groups ahead, the
//     next step's A fragments during the step's last groups, so no group
//     waits for LDS.  The slice's second step, once past its last read of
//     the slice's buffers, waits for every wave (one barrier per slice) and
//     then reads the next slice's first fragments.
//   * an LDS row holds 64 k values (8 chunks of 16 bytes); the chunk index
//     is XOR-swizzled with (row >> 1) & 7: the 16 lanes of a phase of a
//     fragment read (rows r .. r+15 at one chunk, 256 bytes of LDS banks)
//     then hit 16 different 16-byte bank groups.
//   * both operands are K-contiguous (A [M, K], W [N, K]), so both
//     fragments are plain 16-byte LDS reads.  W is the MFMA's first operand
//     and A the second: the accumulator block is then C^T, and each lane
//     holds one row m of C with 4 consecutive columns n per block.
//   * when K is a multiple of 128 the loads need no per-lane k check: a
//     slice's k offset is the scalar offset of its loads.  A piece's row
//     stays in the lane offset, which the buffer's range check covers (the
//     scalar offset is not checked), so rows past M or N read as zero.
//   * the bias is the accumulators' starting value, so the matrix cores add
//     the products to it; the epilogue in registers applies GELU (erfc from
//     Abramowitz and Stegun 7.1.26, rearranged so one form serves both
//     signs) and rounds to bf16; then each wave stages its 64 x 128 bf16
//     part in LDS (rows of 256 bytes, 16-byte chunks XOR-swizzled with
//     row & 15, the 8-byte halves of a chunk swapped in rows with bit 4 set)
//     and writes C in whole 16-byte pieces, 4 rows of 256 bytes per wave
//     instruction.
//   * tile order: about 256 consecutive workgroups run together, dealt
//     round-robin to the 8 XCDs; each such window takes a 16 x 16 block of
//     tiles and each XCD a 4 x 8 part of it, so tiles share operand slices
//     in the XCD's L2 and across the window in the memory-side cache.
//   * small problems (up to 128 tiles of 256 x 256) run a variant on
//     128 x 256 tiles, 4 waves and one 48 KiB slice buffer per workgroup, two
//     workgroups per CU: twice the workgroups for the same problem (see
//     gemm_kernel_small below).
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
constexpr int kWaves = 8;
constexpr int kRowBytes = kBK * 2;                    // 128 bytes of k per LDS row
constexpr int kSliceBytes = kBM * kRowBytes;          // 32 KiB per operand slice
constexpr int kLoadsPerWave = kSliceBytes / (kWaves * 1024);   // 4 per operand
constexpr uint32_t kOut = 0x80000000u;                // a buffer offset past any range

static_assert(kSliceBytes % (kWaves * 1024) == 0, "a slice must split evenly over the waves");

G_INLINE __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

G_INLINE f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

G_INLINE u32x4 lds_read16(const lds_u8* p) { return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p); }

// GELU(z) = z Phi(z), Phi(z) = erfc(-z / sqrt 2) / 2, with erfc by Abramowitz
// and Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erfc(x) ~ t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) exp(-x^2),
// t = 1 / (1 + p x), for x >= 0 (absolute error below 1.5e-7), and
// erfc(-x) = 2 - erfc(x).  With a = |z| and h = erfc(a / sqrt 2) / 2 both
// signs reduce to one form: z >= 0 gives z (1 - h), z < 0 gives z h, and
// both equal max(z, 0) - a h.  The 1/sqrt(2) and the 1/2 are folded into
// the constants: t = 1 / (1 + (p / sqrt 2) a), exp(-a^2 / 2) =
// exp2(-a^2 log2(e) / 2), coefficients a_i / 2.  Over z in [-12, 12] it stays
// within 4.3e-7 of the exact GELU in fp32 (at most 1.7e-4 relative where
// |GELU| > 1e-3), far below the bf16 rounding of the output.
G_INLINE float gelu(float z) {
  const float a = __builtin_fabsf(z);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.23164190f, a, 1.0f));   // p / sqrt 2, p = 0.3275911
  const float e = __builtin_amdgcn_exp2f((a * -0.72134752044448170f) * a);        // -log2(e) / 2
  float q = __builtin_fmaf(t, 0.5307027145f, -0.7265760135f);                   // a5/2, a4/2
  q = __builtin_fmaf(t, q, 0.7107068705f);                                     // a3/2
  q = __builtin_fmaf(t, q, -0.142248368f);                                     // a2/2
  q = __builtin_fmaf(t, q, 0.127414796f);                                      // a1/2
  return __builtin_fmaf(-(a * e), q * t, __builtin_fmaxf(z, 0.0f));
}

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

// KFULL: K is a multiple of 2 * kBK, so every slice the loop computes lies
// inside K and the loads need no per-lane k check (the k offset of a slice
// is the scalar offset of the load; the row of a piece is in the lane
// offset, where the range check sees it).
template <int EPI, bool KFULL>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
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
  const int wm = wave >> 1, wn = wave & 1;             // this wave's 64 x 128 part of the tile

  // ---- tile of this workgroup ---------------------------------------------
  // Workgroups start in index order, dealt round-robin to the 8 XCDs (b % 8),
  // 32 at a time per XCD (one per CU), so about 256 consecutive indices run
  // together.  Each such window takes a 16 x 16 block of tiles, and XCD x
  // a 4 x 8 part of it: the 32 tiles on one XCD share 4 row slices of A and 8
  // of W in its L2, and the 256 tiles of a window share 16 + 16 in the
  // memory-side cache.  Windows run along a band of 16 tile-rows, so the next
  // window keeps the band's A.  Partial windows and partial blocks at the
  // edges take their tiles in plain order.
  const int nt = (int)gridDim.x, b = (int)blockIdx.x;
  const int full = nt & ~255;
  const int t = b < full ? (b & ~255) + 32 * (b & 7) + ((b >> 3) & 31) : b;
  const int band = 16 * p.tiles_n;                     // tiles in a band of 16 tile-rows
  const int br = t / band, hm = min(16, p.tiles_m - 16 * br);
  const int ub = t - br * band;                        // index inside the band
  const int bc = ub / (16 * hm), hn = min(16, p.tiles_n - 16 * bc);
  const int v = ub - bc * 16 * hm;                     // index inside the hm x hn block
  int tm, tn;
  if (hm == 16 && hn == 16) {
    const int part = v >> 5, w = v & 31;               // 4 x 8 part of the block, tile in it (column-major)
    tm = 16 * br + 4 * (part >> 1) + (w & 3);
    tn = 16 * bc + 8 * (part & 1) + (w >> 2);
  } else {
    tm = 16 * br + v % hm;
    tn = 16 * bc + v / hm;
  }
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- operand loads: HBM -> LDS ----------------------------------------------
  // Load t of a wave fills LDS bytes [(wave*4 + t) KiB, +1 KiB): chunk index
  // idx = (wave*4 + t)*64 + lane, row idx / 8, swizzled chunk idx % 8, which
  // holds logical chunk (idx % 8) ^ ((row >> 1) & 7): k = 8 * that chunk.
  const uint32_t a_rows = (uint32_t)min(kBM, M - m0), w_rows = (uint32_t)min(kBN, N - n0);
  const __amdgpu_buffer_rsrc_t ars = rsrc(p.a + (size_t)m0 * K, a_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wrs = rsrc(p.w + (size_t)n0 * K, w_rows * (uint32_t)K * 2u);
  // Piece s of a wave covers rows row0 + 8 s: the swizzle term (row >> 1) & 7
  // then differs between even and odd s only (by 4), so two k offsets serve
  // all pieces.  The row of a piece stays in the lane offset (one register
  // per piece): the buffer's range check covers the lane offset and not the
  // scalar one, and rows past M or N must fall out of range.
  const int row0 = wave * kLoadsPerWave * 8 + (lane >> 3);
  int ld_k[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) ld_k[par] = 8 * ((lane & 7) ^ (((row0 >> 1) + 4 * par) & 7));
  uint32_t ld_off[kLoadsPerWave];
#pragma unroll
  for (int s = 0; s < kLoadsPerWave; ++s) ld_off[s] = (uint32_t)((row0 + 8 * s) * K + ld_k[s & 1]) * 2u;
  // A slice moves global -> VGPRs -> LDS: each wave loads its 8 pieces of
  // slice j+2 into registers during slice j and writes them to LDS during
  // slice j+1, so the loads spread over the slice and still have a slice of
  // lead.
  u32x4 ra[kLoadsPerWave], rw[kLoadsPerWave];
  auto gload = [&](__amdgpu_buffer_rsrc_t rs, int s, int k0) -> u32x4 {
    if constexpr (KFULL) {
      // the loads of the two slices past K (issued by the last two slices,
      // never used) are sent out of range through the lane offset, which is
      // what the buffer's range check covers, so nothing is read
      const bool in = k0 < K;
      return __builtin_amdgcn_raw_buffer_load_b128(rs, in ? ld_off[s] : kOut, in ? (uint32_t)k0 * 2u : 0u, 0);
    } else {
      const int k = k0 + ld_k[s & 1];
      const uint32_t off = k < K ? (uint32_t)((row0 + 8 * s) * K + k) * 2u : kOut;
      return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  };
  auto swrite = [&](lds_u8* buf, int s, u32x4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(buf + (wave * kLoadsPerWave + s) * 1024 + lane * 16) = v;
  };
  // piece q of 8 (0-3 A, 4-7 W): write the staged value into the next
  // slice's buffer, then load the same piece of the slice after it
  auto stage_piece = [&](lds_u8* nabuf, lds_u8* nwbuf, int q, int k2) __attribute__((always_inline)) {
    if (q < kLoadsPerWave) {
      swrite(nabuf, q, ra[q]);
      ra[q] = gload(ars, q, k2);
    } else {
      swrite(nwbuf, q - kLoadsPerWave, rw[q - kLoadsPerWave]);
      rw[q - kLoadsPerWave] = gload(wrs, q - kLoadsPerWave, k2);
    }
  };

  // ---- fragment reads: lane l reads row l % 16 of a 16-row block, k chunk
  // 4*ks + l / 16 of the slice (k32 step ks), at its swizzled place.
  int rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd[ks] = (lane & 15) * kRowBytes + (((4 * ks + (lane >> 4)) ^ ((lane >> 1) & 7)) << 4);
  const int a_base = wm * 64 * kRowBytes, w_base = wn * 128 * kRowBytes;

  // Accumulators start at the bias (register r of a lane in column block nb
  // is column nb*16 + 4*(lane / 16) + r, for every row block), so the matrix
  // cores add the products on top and no epilogue add is left.
  f32x4 acc[4][8];
  {
    const int h4 = 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t brs = rsrc(p.bias, EPI != 0 ? (uint32_t)N * 4u : 0u);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 bv = {};
      asm volatile("" : "+v"(bv));   // distinct starting values: each block accumulates in place
      if constexpr (EPI != 0) {
        const int n = n0 + wn * 128 + nb * 16 + h4;
        bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, n < N ? (uint32_t)n * 4u : kOut, 0, 0));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = bv;
    }
  }

  auto rda = [&](const lds_u8* abuf, int ks, int mb) { return lds_read16(abuf + a_base + mb * 16 * kRowBytes + rd[ks]); };
  auto rdw = [&](const lds_u8* wbuf, int ks, int nb) { return lds_read16(wbuf + w_base + nb * 16 * kRowBytes + rd[ks]); };
  // A k32 step is 8 groups of 4 MFMAs (group nb: the W fragment nb against
  // the 4 A fragments).  W fragments are read two groups ahead into a ring of
  // 4 (8 groups a step keep its places fixed from step to step); the next
  // step's A fragments go into the other of two A sets during the step's
  // last groups.  A slice (two steps): step 0 stages the 4 A pieces, one
  // every other group; step 1 stages the 4 W pieces in groups 0-3 and, after
  // group 5 (its last reads of this slice's buffers), waits for its LDS
  // traffic and every wave, then reads the next slice's first fragments
  // during groups 6 and 7.
  u32x4 af[2][4], wr[4];
  auto step = [&](const lds_u8* abuf, const lds_u8* wbuf, int ks, int cur, const lds_u8* nabuf, const lds_u8* nwbuf,
                  bool last, lds_u8* sabuf, lds_u8* swbuf, int k2) __attribute__((always_inline)) {
    // on entry: af[cur] holds this step's A fragments, wr[0], wr[1] its W fragments 0 and 1
    const lds_u8* na = last ? nabuf : abuf;
    const lds_u8* nw = last ? nwbuf : wbuf;
    const int nks = last ? 0 : 1;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      if (last && nb == 6) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      // the W fragment two groups ahead (this step's, or the next step's 0 and 1)
      if (nb + 2 < 8) wr[(nb + 2) % 4] = rdw(wbuf, ks, nb + 2);
      else wr[(nb + 2) % 4] = rdw(nw, nks, nb - 6);
      // the next step's A fragments, during groups 4-7 (after the barrier when the step is the slice's last)
      if (nb >= 4 && (!last || nb >= 6)) {
        if (last) {
          af[cur ^ 1][2 * (nb - 6)] = rda(na, nks, 2 * (nb - 6));
          af[cur ^ 1][2 * (nb - 6) + 1] = rda(na, nks, 2 * (nb - 6) + 1);
        } else {
          af[cur ^ 1][nb - 4] = rda(na, nks, nb - 4);
        }
      }
      if (ks == 0 && (nb & 1) == 0) stage_piece(sabuf, swbuf, nb >> 1, k2);   // A pieces: every other group of step 0
      if (ks == 1 && nb < 4) stage_piece(sabuf, swbuf, 4 + nb, k2);           // W pieces: groups 0-3 of step 1
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma(wr[nb % 4], af[cur][mb], acc[mb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute = [&](const lds_u8* abuf, const lds_u8* wbuf, lds_u8* nabuf, lds_u8* nwbuf, int k2) __attribute__((always_inline)) {
    step(abuf, wbuf, 0, 0, nabuf, nwbuf, false, nabuf, nwbuf, k2);
    step(abuf, wbuf, 1, 1, nabuf, nwbuf, true, nabuf, nwbuf, k2);
  };

  // ---- main loop: two slices per iteration, one per buffer --------------------
  // The slice count is rounded up to even (a slice past K reads as zeros),
  // so the loop has one exit and the accumulators one loop-carried copy.
  // The last two slices issue loads past K, which only write zeros into
  // LDS; the barrier after the loop waits for them.
  const int nk = ((K + kBK - 1) / kBK + 1) & ~1;
#pragma unroll
  for (int s2 = 0; s2 < kLoadsPerWave; ++s2) {
    ra[s2] = gload(ars, s2, 0);
    rw[s2] = gload(wrs, s2, 0);
  }
#pragma unroll
  for (int s2 = 0; s2 < kLoadsPerWave; ++s2) {
    swrite(A0, s2, ra[s2]);
    swrite(W0, s2, rw[s2]);
  }
#pragma unroll
  for (int s2 = 0; s2 < kLoadsPerWave; ++s2) ra[s2] = gload(ars, s2, kBK);
#pragma unroll
  for (int s2 = 0; s2 < kLoadsPerWave; ++s2) rw[s2] = gload(wrs, s2, kBK);
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) af[0][mb] = rda(A0, 0, mb);
  wr[0] = rdw(W0, 0, 0);
  wr[1] = rdw(W0, 0, 1);
  for (int j = 0; j < nk; j += 2) {
    compute(A0, W0, A1, W1, (j + 2) * kBK);   // slice j; writes slice j+1, loads slice j+2
    compute(A1, W1, A0, W0, (j + 3) * kBK);   // slice j+1; writes slice j+2, loads slice j+3
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // every wave is done reading the slices: LDS is free for the output.  The
  // scheduling barriers keep the accumulator reads of the epilogue below
  // it (hoisted above, all 256 values would sit in VGPRs at once).
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue -------------------------------------------------------------
  // Lane l holds, for block (mb, nb), row m = mb*16 + l % 16 of the wave's
  // 64 x 128 part and columns nb*16 + 4*(l / 16) + r for register r.  Each
  // wave stages its part in one half of a 32 KiB LDS object.
  lds_u8* const stage = (wave >> 1 == 0 ? A0 : wave >> 1 == 1 ? W0 : wave >> 1 == 2 ? A1 : W1) + (wave & 1) * 16384;
  // the lane index again, from the execution mask (all lanes are active),
  // so no register holds it through the loop and the epilogue's addresses
  // are computed here
  int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(el));
  const int g4 = el >> 4, ml = el & 15;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = mb * 16 + ml;
      const float v0 = activation<EPI>(acc[mb][nb][0]);
      const float v1 = activation<EPI>(acc[mb][nb][1]);
      const float v2 = activation<EPI>(acc[mb][nb][2]);
      const float v3 = activation<EPI>(acc[mb][nb][3]);
      u32x2 pk;
      pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v0, v1}, bf16x2));
      pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v2, v3}, bf16x2));
      const int chunk = nb * 2 + (g4 >> 1);            // 16-byte chunk of the 256-byte row
      const int h = g4 & 1;                            // 8-byte half of the chunk
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * (h ^ ((row >> 4) & 1))) = pk;
      if (mb & 1) __builtin_amdgcn_sched_barrier(0);   // two blocks at a time: no hoisting of every block's values
    }
  }
  // each wave reads back only what it wrote
  const uint32_t c_rows = (uint32_t)min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t crs = rsrc(p.c + (size_t)m0 * N, c_rows * (uint32_t)N * 2u);
  const int c = el & 15;
  const int n = n0 + wn * 128 + c * 8;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int row = it * 4 + (el >> 4);
    u32x4 v = lds_read16(stage + row * 256 + ((c ^ (row & 15)) << 4));
    if ((it >> 2) & 1) v = (u32x4){v[2], v[3], v[0], v[1]};   // rows with bit 4 set hold their halves swapped
    const uint32_t off = n < N ? ((uint32_t)(wm * 64 + row) * (uint32_t)N + (uint32_t)n) * 2u : kOut;
    __builtin_amdgcn_raw_buffer_store_b128(v, crs, off, 0, 0);
  }
}


// The small-problem variant: a workgroup of 4 waves (64 x 128 each) computes
// a 128 x 256 tile with one 48 KiB slice buffer, so two workgroups share a CU
// and a problem of up to 128 tiles of 256 x 256 fills twice as many
// workgroups.  Same operand order, fragment layout, swizzle, accumulation
// order and epilogue as the main kernel, so C is bit-identical.
constexpr int kSBM = 128, kSBN = 256;
constexpr int kSWaves = 4;
constexpr int kSABytes = kSBM * kRowBytes;            // 16 KiB A slice
constexpr int kSWBytes = kSBN * kRowBytes;            // 32 KiB W slice
constexpr int kSAPieces = kSABytes / (kSWaves * 1024);   // 4 per wave
constexpr int kSWPieces = kSWBytes / (kSWaves * 1024);   // 8 per wave

template <int EPI, bool KFULL>
__global__ void __launch_bounds__(kSWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_kernel_small(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds[kSABytes];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds[kSWBytes];
  lds_u8* const AL = (lds_u8*)a_lds;
  lds_u8* const WL = (lds_u8*)w_lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;             // this wave's 64 x 128 part of the 128 x 256 tile

  // ---- tile: windows of 512 consecutive workgroups (two per CU), dealt
  // round-robin to the 8 XCDs; a window takes a 32 x 16 block of 128 x 256
  // tiles and XCD x an 8 x 8 part of it (partial windows and blocks in plain
  // order).
  const int nt = (int)gridDim.x, b = (int)blockIdx.x;
  const int full = nt & ~511;
  const int t = b < full ? (b & ~511) + 64 * (b & 7) + ((b >> 3) & 63) : b;
  const int band = 32 * p.tiles_n;                     // tiles in a band of 32 tile-rows
  const int br = t / band, hm = min(32, p.tiles_m - 32 * br);
  const int ub = t - br * band;
  const int bc = ub / (16 * hm), hn = min(16, p.tiles_n - 16 * bc);
  const int v = ub - bc * 16 * hm;
  int tm, tn;
  if (hm == 32 && hn == 16) {
    const int part = v >> 6, w = v & 63;               // 8 x 8 part of the block, tile in it
    tm = 32 * br + 8 * (part >> 1) + (w & 7);
    tn = 16 * bc + 8 * (part & 1) + (w >> 3);
  } else {
    tm = 32 * br + v % hm;
    tn = 16 * bc + v / hm;
  }
  const int m0 = tm * kSBM, n0 = tn * kSBN;
  const int M = p.M, N = p.N, K = p.K;

  const uint32_t a_rows = (uint32_t)min(kSBM, M - m0), w_rows = (uint32_t)min(kSBN, N - n0);
  const __amdgpu_buffer_rsrc_t ars = rsrc(p.a + (size_t)m0 * K, a_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wrs = rsrc(p.w + (size_t)n0 * K, w_rows * (uint32_t)K * 2u);
  // piece s of A covers rows ra0 + 8 s, of W rows rw0 + 8 s
  const int ra0 = wave * kSAPieces * 8 + (lane >> 3), rw0 = wave * kSWPieces * 8 + (lane >> 3);
  int lka[2], lkw[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    lka[par] = 8 * ((lane & 7) ^ (((ra0 >> 1) + 4 * par) & 7));
    lkw[par] = 8 * ((lane & 7) ^ (((rw0 >> 1) + 4 * par) & 7));
  }
  // lane offset of each piece, its row included (the range check covers the
  // lane offset only, and rows past M or N must fall out of range)
  uint32_t loa[kSAPieces], low[kSWPieces];
#pragma unroll
  for (int s = 0; s < kSAPieces; ++s) loa[s] = (uint32_t)((ra0 + 8 * s) * K + lka[s & 1]) * 2u;
#pragma unroll
  for (int s = 0; s < kSWPieces; ++s) low[s] = (uint32_t)((rw0 + 8 * s) * K + lkw[s & 1]) * 2u;
  auto gload = [&](__amdgpu_buffer_rsrc_t rs, const uint32_t* lo, const int (&lk)[2], int row0, int s, int k0) -> u32x4 {
    if constexpr (KFULL) {
      const bool in = k0 < K;
      return __builtin_amdgcn_raw_buffer_load_b128(rs, in ? lo[s] : kOut, in ? (uint32_t)k0 * 2u : 0u, 0);
    } else {
      const int k = k0 + lk[s & 1];
      const uint32_t off = k < K ? (uint32_t)((row0 + 8 * s) * K + k) * 2u : kOut;
      return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  };
  u32x4 ra[kSAPieces], rw[kSWPieces];
  auto load_slice = [&](int q, int k0) __attribute__((always_inline)) {   // piece q of 12 (0-3 A, 4-11 W)
    if (q < kSAPieces) ra[q] = gload(ars, loa, lka, ra0, q, k0);
    else rw[q - kSAPieces] = gload(wrs, low, lkw, rw0, q - kSAPieces, k0);
  };
  auto write_slice = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kSAPieces; ++s)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(AL + (wave * kSAPieces + s) * 1024 + lane * 16) = ra[s];
#pragma unroll
    for (int s = 0; s < kSWPieces; ++s)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(WL + (wave * kSWPieces + s) * 1024 + lane * 16) = rw[s];
  };

  int rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd[ks] = (lane & 15) * kRowBytes + (((4 * ks + (lane >> 4)) ^ ((lane >> 1) & 7)) << 4);
  const int a_base = wm * 64 * kRowBytes, w_base = wn * 128 * kRowBytes;

  f32x4 acc[4][8];
  {
    const int h4 = 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t brs = rsrc(p.bias, EPI != 0 ? (uint32_t)N * 4u : 0u);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 bv = {};
      asm volatile("" : "+v"(bv));
      if constexpr (EPI != 0) {
        const int n = n0 + wn * 128 + nb * 16 + h4;
        bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, n < N ? (uint32_t)n * 4u : kOut, 0, 0));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = bv;
    }
  }

  auto rda = [&](int ks, int mb) { return lds_read16(AL + a_base + mb * 16 * kRowBytes + rd[ks]); };
  auto rdw = [&](int ks, int nb) { return lds_read16(WL + w_base + nb * 16 * kRowBytes + rd[ks]); };
  u32x4 af[2][4], wr[4];
  // One LDS slice buffer.  A slice (k 64): wait for every wave's pieces,
  // read the first fragments, run two k32 steps of 8 groups of 4 MFMAs (W
  // fragments two groups ahead, the second step's A fragments during the
  // first step's last groups), wait for every wave to finish reading, write
  // the next slice's pieces (loaded a slice earlier) and load the one after.
  const int nk = (K + kBK - 1) / kBK;
#pragma unroll
  for (int q = 0; q < kSAPieces + kSWPieces; ++q) load_slice(q, 0);
  write_slice();
#pragma unroll
  for (int q = 0; q < kSAPieces + kSWPieces; ++q) load_slice(q, kBK);
  for (int j = 0; j < nk; ++j) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[0][mb] = rda(0, mb);
    wr[0] = rdw(0, 0);
    wr[1] = rdw(0, 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        if (nb + 2 < 8) wr[(nb + 2) % 4] = rdw(ks, nb + 2);
        else if (ks == 0) wr[(nb + 2) % 4] = rdw(1, nb - 6);
        if (ks == 0 && nb >= 4) af[1][nb - 4] = rda(1, nb - 4);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma(wr[nb % 4], af[ks][mb], acc[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    write_slice();   // slice j+1 (past K: zeros, never read)
#pragma unroll
    for (int q = 0; q < kSAPieces + kSWPieces; ++q) load_slice(q, (j + 2) * kBK);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue: each wave stages its 64 x 128 part in two rounds of 32 rows
  // (8 KiB per wave per round) and stores whole 16-byte pieces.
  lds_u8* const stage = (wave < 2 ? AL : WL) + (wave & 1) * 8192;
  int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(el));
  const int g4 = el >> 4, ml = el & 15;
  const uint32_t c_rows = (uint32_t)min(kSBM, M - m0);
  const __amdgpu_buffer_rsrc_t crs = rsrc(p.c + (size_t)m0 * N, c_rows * (uint32_t)N * 2u);
  const int c = el & 15;
  const int n = n0 + wn * 128 + c * 8;
#pragma unroll
  for (int rnd = 0; rnd < 2; ++rnd) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        const int mb = 2 * rnd + mh;
        const int row = mh * 16 + ml;                    // row within the round's 32
        const float v0 = activation<EPI>(acc[mb][nb][0]);
        const float v1 = activation<EPI>(acc[mb][nb][1]);
        const float v2 = activation<EPI>(acc[mb][nb][2]);
        const float v3 = activation<EPI>(acc[mb][nb][3]);
        u32x2 pk;
        pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v0, v1}, bf16x2));
        pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v2, v3}, bf16x2));
        const int chunk = nb * 2 + (g4 >> 1);
        const int h = g4 & 1;
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * (h ^ ((row >> 4) & 1))) = pk;
      }
      if (nb & 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 4 + (el >> 4);
      u32x4 vv = lds_read16(stage + row * 256 + ((c ^ (row & 15)) << 4));
      if ((it >> 2) & 1) vv = (u32x4){vv[2], vv[3], vv[0], vv[1]};
      const uint32_t off = n < N ? ((uint32_t)(wm * 64 + rnd * 32 + row) * (uint32_t)N + (uint32_t)n) * 2u : kOut;
      __builtin_amdgcn_raw_buffer_store_b128(vv, crs, off, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of this round done before the next round's writes
  }
}

// ---- 4-wave variant: one workgroup of 4 waves per CU, 128 x 128 per wave ----
// A 256 x 256 tile; each wave owns 128 x 128 of it as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators a lane, one wave per SIMD).
// The operand slices (k 64) reach LDS straight from memory (buffer_load ...
// lds, no VGPR staging), double-buffered; one barrier per slice.  K must be a
// multiple of kBK, so no k chunk of a loaded slice lies past K and the loads
// need no per-lane k check (a check in every load measured 5 % slower than
// the 8-wave kernel on K = 4104: the 4-wave loop has no VALU to hide it).
constexpr int k4Waves = 4;
constexpr int k4Pieces = kSliceBytes / (k4Waves * 1024);   // 8 pieces of 1 KiB per operand per wave

// Raw buffer descriptor as four dwords (base, size in bytes, format word), for
// the inline-asm loads below.
G_INLINE u32x4 rsrc4(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)(size_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nbytes, 0x00020000u};
}

// One 1 KiB piece HBM -> LDS: lane l's 16 bytes at lane offset off (the part
// the range check covers) plus the scalar offset soff land at dst + 16 l.
G_INLINE void load_lds(u32x4 rs, lds_u8* dst, uint32_t off, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("" : "+s"(soff));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}

template <int EPI>
__global__ void __launch_bounds__(k4Waves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel4(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[4 * kSliceBytes];   // A0 W0 A1 W1
  lds_u8* const L = (lds_u8*)lds_all;
  lds_u8* const A0 = L;
  lds_u8* const W0 = L + kSliceBytes;
  lds_u8* const A1 = L + 2 * kSliceBytes;
  lds_u8* const W1 = L + 3 * kSliceBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;             // this wave's 128 x 128 part of the tile

  // tile of this workgroup: the same order as gemm_kernel
  const int nt = (int)gridDim.x, b = (int)blockIdx.x;
  const int full = nt & ~255;
  const int t = b < full ? (b & ~255) + 32 * (b & 7) + ((b >> 3) & 31) : b;
  const int band = 16 * p.tiles_n;
  const int br = t / band, hm = min(16, p.tiles_m - 16 * br);
  const int ub = t - br * band;
  const int bc = ub / (16 * hm), hn = min(16, p.tiles_n - 16 * bc);
  const int v = ub - bc * 16 * hm;
  int tm, tn;
  if (hm == 16 && hn == 16) {
    const int part = v >> 5, w = v & 31;
    tm = 16 * br + 4 * (part >> 1) + (w & 3);
    tn = 16 * bc + 8 * (part & 1) + (w >> 2);
  } else {
    tm = 16 * br + v % hm;
    tn = 16 * bc + v / hm;
  }
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- operand pieces: piece q of wave w covers rows 64 w + 8 q .. + 7 of
  // the slice; lane l fetches row 64 w + 8 q + l / 8 into LDS slot l % 8 of
  // that row, which holds logical chunk (l % 8) ^ ((row >> 1) & 7).  The row
  // stays in the lane offset, so rows past M or N fall out of the range.
  const uint32_t a_rows = (uint32_t)min(kBM, M - m0), w_rows = (uint32_t)min(kBN, N - n0);
  const u32x4 ars = rsrc4(p.a + (size_t)m0 * K, a_rows * (uint32_t)K * 2u);
  const u32x4 wrs = rsrc4(p.w + (size_t)n0 * K, w_rows * (uint32_t)K * 2u);
  const u32x4 ars0 = (u32x4){ars[0], ars[1], 0u, ars[3]};   // no bytes: every load out of range
  const u32x4 wrs0 = (u32x4){wrs[0], wrs[1], 0u, wrs[3]};
  // (the logical chunk differs between even and odd pieces only)
  uint32_t loff[k4Pieces];
  int lk[2];
  {
    const int row0 = wave * k4Pieces * 8 + (lane >> 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) lk[par] = 8 * ((lane & 7) ^ (((row0 >> 1) + 4 * par) & 7));
#pragma unroll
    for (int q = 0; q < k4Pieces; ++q) loff[q] = (uint32_t)((row0 + 8 * q) * K + lk[q & 1]) * 2u;
  }
  const int wofs = wave * k4Pieces * 1024;
  // piece i of 16 (0-7 A, 8-15 W) of slice s into the buffers ab / wb
  auto load_piece = [&](int i, int s, lds_u8* ab, lds_u8* wb) __attribute__((always_inline)) {
    const bool in = s * kBK < K;
    const int q = i % k4Pieces;
    const uint32_t off = loff[q];
    if (i < k4Pieces)
      load_lds(in ? ars : ars0, ab + wofs + q * 1024, off, (uint32_t)(s * kBK) * 2u);
    else
      load_lds(in ? wrs : wrs0, wb + wofs + q * 1024, off, (uint32_t)(s * kBK) * 2u);
  };

  // ---- fragment reads: lane l reads row l % 16 of a 16-row block, k chunk
  // 4 ks + l / 16 of the slice, at its swizzled place
  int rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd[ks] = (lane & 15) * kRowBytes + (((4 * ks + (lane >> 4)) ^ ((lane >> 1) & 7)) << 4);
  const int a_base = wm * 128 * kRowBytes, w_base = wn * 128 * kRowBytes;
  auto rda = [&](const lds_u8* ab, int ks, int mb) { return lds_read16(ab + a_base + mb * 16 * kRowBytes + rd[ks]); };
  auto rdw = [&](const lds_u8* wb, int ks, int nb) { return lds_read16(wb + w_base + nb * 16 * kRowBytes + rd[ks]); };

  // accumulators start at the bias (column nb*16 + 4*(lane/16) + r of block nb)
  f32x4 acc[8][8];
  {
    const int h4 = 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t brs = rsrc(p.bias, EPI != 0 ? (uint32_t)N * 4u : 0u);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 bv = {};
      asm volatile("" : "+v"(bv));
      if constexpr (EPI != 0) {
        const int n = n0 + wn * 128 + nb * 16 + h4;
        bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, n < N ? (uint32_t)n * 4u : kOut, 0, 0));
      }
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = bv;
    }
  }

  // A k32 step: 64 MFMAs (W fragment nb against A fragment mb), with the
  // next step's 16 fragment reads spread one per 4 MFMAs and, when `loads`,
  // this wave's 16 pieces of the slice after next, one per 4 MFMAs.
  u32x4 af[2][8], wf[2][8];
  auto step = [&](int cur, const lds_u8* nab, const lds_u8* nwb, int nks, bool loads, int ls, lds_u8* lab,
                  lds_u8* lwb) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 64; ++g) {
      const int nb = g >> 3, mb = g & 7;
      if ((g & 3) == 0) {
        const int r = g >> 2;   // 0..15: next A fragments 0-7, then W 0-7
        if (r < 8) af[cur ^ 1][r] = rda(nab, nks, r);
        else wf[cur ^ 1][r - 8] = rdw(nwb, nks, r - 8);
      }
      if (loads && (g & 3) == 2) load_piece(g >> 2, ls, lab, lwb);
      acc[mb][nb] = mfma(wf[cur][nb], af[cur][mb], acc[mb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // vmcnt(0) lgkmcnt(0) where the compiler sees it (0x70: expcnt left
  // alone), so no read is pending across the loop's back edge and no step
  // waits for the previous one's reads, then the barrier; scheduling fences
  // keep every memory operation on its side
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x70);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop ---------------------------------------------------------------
  // Slice s sits in buffer s % 2.  Step 0 of slice s reads its step-1
  // fragments; then every wave waits for its pieces of slice s+1 and for the
  // others (barrier: buffer s % 2 is no longer read, slice s+1 has landed);
  // step 1 reads slice s+1's step-0 fragments and loads slice s+2 into
  // buffer s % 2.  The loop runs from barrier to barrier (two slices an
  // iteration), so nothing is in flight across its back edge.  The slice
  // count is rounded up to even (a slice past K reads as zeros and adds
  // exactly nothing), so the loop and its tail are one code path.
  const int nk = ((K + kBK - 1) / kBK + 1) & ~1;
#pragma unroll
  for (int i = 0; i < 2 * k4Pieces; ++i) load_piece(i, 0, A0, W0);
#pragma unroll
  for (int i = 0; i < 2 * k4Pieces; ++i) load_piece(i, 1, A1, W1);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // slice 0's pieces
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 8; ++r) af[0][r] = rda(A0, 0, r);
#pragma unroll
  for (int r = 0; r < 8; ++r) wf[0][r] = rdw(W0, 0, r);
  step(0, A0, W0, 1, false, 0, A0, W0);   // slice 0, step 0
  sync();
  int s = 0;
  for (; s + 2 < nk; s += 2) {
    step(1, A1, W1, 0, true, s + 2, A0, W0);   // slice s, step 1
    step(0, A1, W1, 1, false, 0, A1, W1);      // slice s+1, step 0
    sync();
    step(1, A0, W0, 0, true, s + 3, A1, W1);   // slice s+1, step 1
    step(0, A0, W0, 1, false, 0, A0, W0);      // slice s+2, step 0
    sync();
  }
  step(1, A1, W1, 0, true, s + 2, A0, W0);     // slice nk-2, step 1
  step(0, A1, W1, 1, false, 0, A1, W1);        // slice nk-1, step 0
  sync();
  step(1, A0, W0, 0, false, 0, A1, W1);        // slice nk-1, step 1 (its reads are not used)
  // every wave is done with LDS: it takes the output
  __builtin_amdgcn_sched_barrier(0);
  sync();
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue: each wave stages its 128 x 128 bf16 part in 32 KiB of LDS
  // (rows of 256 bytes, chunks XOR-swizzled with row & 15, the 8-byte halves
  // of a chunk swapped in rows with bit 4 set) and writes C in 16-byte pieces
  lds_u8* const stage = L + wave * 32768;
  int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(el));
  const int g4 = el >> 4, ml = el & 15;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int row = mb * 16 + ml;
      const float v0 = activation<EPI>(acc[mb][nb][0]);
      const float v1 = activation<EPI>(acc[mb][nb][1]);
      const float v2 = activation<EPI>(acc[mb][nb][2]);
      const float v3 = activation<EPI>(acc[mb][nb][3]);
      u32x2 pk;
      pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v0, v1}, bf16x2));
      pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v2, v3}, bf16x2));
      const int chunk = nb * 2 + (g4 >> 1);
      const int h = g4 & 1;
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * (h ^ ((row >> 4) & 1))) = pk;
      if (mb & 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint32_t c_rows = (uint32_t)min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t crs = rsrc(p.c + (size_t)m0 * N, c_rows * (uint32_t)N * 2u);
  const int c = el & 15;
  const int n = n0 + wn * 128 + c * 8;
#pragma unroll
  for (int it = 0; it < 32; ++it) {
    const int row = it * 4 + (el >> 4);
    u32x4 val = lds_read16(stage + row * 256 + ((c ^ (row & 15)) << 4));
    if ((it >> 2) & 1) val = (u32x4){val[2], val[3], val[0], val[1]};
    const uint32_t off = n < N ? ((uint32_t)(wm * 128 + row) * (uint32_t)N + (uint32_t)n) * 2u : kOut;
    __builtin_amdgcn_raw_buffer_store_b128(val, crs, off, 0, 0);
  }
}

// Up to 128 tiles of 256 x 256 (at most half the CUs busy) the small-problem
// kernel runs, on twice as many 128 x 256 tiles: measured 8-30 % faster there,
// and 5-15 % slower from 192 tiles up.
hipError_t launch_gemm(int epi, const GemmParams& prm, hipStream_t stream) {
  GemmParams p = prm;
  const long long big_tiles = (long long)((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN);
  const bool small = big_tiles <= 128;
  p.tiles_m = (p.M + (small ? kSBM : kBM) - 1) / (small ? kSBM : kBM);
  p.tiles_n = (p.N + kBN - 1) / kBN;
  const long long tiles = (long long)p.tiles_m * p.tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)tiles);
  if (small) {
    const dim3 block(kSWaves * 64);
    const bool kfull = p.K % kBK == 0;
    switch (epi) {
      case 0:
        if (kfull) hipLaunchKernelGGL((gemm_kernel_small<0, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((gemm_kernel_small<0, false>), grid, block, 0, stream, p);
        break;
      case 1:
        if (kfull) hipLaunchKernelGGL((gemm_kernel_small<1, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((gemm_kernel_small<1, false>), grid, block, 0, stream, p);
        break;
      default:
        if (kfull) hipLaunchKernelGGL((gemm_kernel_small<2, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((gemm_kernel_small<2, false>), grid, block, 0, stream, p);
        break;
    }
    return hipGetLastError();
  }
  const bool kfull = p.K % (2 * kBK) == 0;
  if (big_tiles >= 256 && p.K % kBK == 0) {
    // at least one tile per CU and K a multiple of 64: the 4-wave kernel
    // (measured 3-5 % faster from 256 tiles up, 6 % slower at 144)
    const dim3 block4(k4Waves * 64);
    switch (epi) {
      case 0: hipLaunchKernelGGL((gemm_kernel4<0>), grid, block4, 0, stream, p); break;
      case 1: hipLaunchKernelGGL((gemm_kernel4<1>), grid, block4, 0, stream, p); break;
      default: hipLaunchKernelGGL((gemm_kernel4<2>), grid, block4, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  const dim3 block(kWaves * 64);
  switch (epi) {
    case 0:
      if (kfull) hipLaunchKernelGGL((gemm_kernel<0, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((gemm_kernel<0, false>), grid, block, 0, stream, p);
      break;
    case 1:
      if (kfull) hipLaunchKernelGGL((gemm_kernel<1, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((gemm_kernel<1, false>), grid, block, 0, stream, p);
      break;
    default:
      if (kfull) hipLaunchKernelGGL((gemm_kernel<2, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((gemm_kernel<2, false>), grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace ttc_gemm



