// Fused attention forward for gfx950 (CDNA4, wave64, MFMA).
//
// Method: TileLang tutorial "Designing high-performance GPU kernels with a
// high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
// section on the fused FlashAttention forward kernel -- each workgroup owns
// a tile of query rows, streams key/value tiles past it, and keeps an online
// softmax (running maximum, running normalisation sum, rescaling factor) so
// the score matrix never leaves the chip; both products run on the matrix
// cores.
//
// Work split and data flow (all of it designed for CDNA4):
//   * workgroup = NW waves; wave w owns 32*QT query rows; the workgroup owns
//     BM = NW*32*QT rows of one (batch, head).
//   * Q: each wave keeps its rows in VGPRs for the whole pass, as the B
//     operand of v_mfma_f32_32x32x16 (8 consecutive head-dim elements per
//     lane), loaded once from HBM.
//   * K/V: BC-key tiles are copied HBM -> LDS with global_load_lds_dwordx4
//     (no VGPR staging), double buffered: the next tile's loads are in
//     flight while the current tile is computed; one barrier per tile.
//   * two workgroups share a CU (<= 256 VGPRs per wave, 2 waves per SIMD) so
//     one wave's softmax VALU work overlaps the other's MFMAs.
//   * scores are computed transposed, S^T = K Q^T, so the accumulator puts
//     one query row per lane (column = lane % 32) and 16 of its keys in the
//     lane's registers; the other 16 keys of that row sit in lane ^ 32.  A
//     row reduction is in-lane work plus one v_permlane32_swap.
//   * O is accumulated transposed too, O^T += V^T P^T: the probabilities
//     feed the B operand straight from the score registers (no LDS round
//     trip), and every accumulator register of a lane belongs to that lane's
//     query row, so the rescale by alpha is lane-local.
//   * the V^T operand is read from the row-major V tile with
//     ds_read_b64_tr_b16 (gfx950 transposing LDS read), so V never needs a
//     transposed copy.
//   * softmax in base 2: p = exp2(s*c - m*c) with c = scale*log2(e) folded
//     into one FMA; LSE = ln2 * (m*c + log2(l)) at the end.
//   * the running maximum m used as the exponent reference is moved (and
//     O, l rescaled by alpha = exp2((m_old - m_new)*c)) only when some row's
//     tile maximum exceeds it by more than a margin (in log2 units); when no
//     row of the wave qualifies, the rescale of O is skipped.  bf16 uses a
//     zero margin: m is the exact running maximum, so a row's largest
//     probability is exactly 1 and survives the bf16 rounding of P without
//     error (this matters on peaky rows).  fp16, with 8 more bits of
//     mantissa for P, keeps a stale reference until a row outgrows it by
//     2^8 (p <= 256).  O / l and LSE do not depend on the reference.
//
// LDS layout of one stage: K tile [BC][D] then V tile [BC][D], bf16/fp16,
// rows of D*2 bytes split in 16-byte chunks.  The chunk index is XOR-swizzled
// per row so the two read patterns are free of bank conflicts:
//   K: chunk ^ (row & 7)      (8 consecutive rows read the same chunk)
//   V: chunk ^ 2*(row & 3)    (4 consecutive rows read one 32-byte segment)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace ttc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Element-type specific pieces: the 32x32x16 MFMA and the fp32 -> 16-bit
// pair conversion (round to nearest even) used for the probabilities.
template <bool BF16>
struct Ops;

template <>
struct Ops<true> {
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
};

template <>
struct Ops<false> {
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
};

// Row reductions across the two lane halves: lanes l and l ^ 32 hold the
// two halves of one query row.  v_permlane32_swap(x, x) gives lanes 0-31
// (own, lane + 32) and lanes 32-63 (lane - 32, own), so combining the two
// results yields the same value in both lanes.
__device__ static inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ static inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ static inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF16, int D, int BC, int QT, int NW, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(AttnParams p) {
  using O = Ops<BF16>;
  constexpr int BM = NW * 32 * QT;             // query rows per workgroup
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = BC * ROW_BYTES;   // one K or V tile
  constexpr int NT = NW * 64;                  // threads per workgroup
  constexpr int PER_W = BC * CPR / 64 / NW;    // 1 KiB direct loads per wave per tile
  constexpr int KB = BC / 32;                  // 32-key blocks per tile
  constexpr int DK = D / 16;                   // k-steps of the score product
  constexpr int DT = D / 32;                   // 32-wide head-dim blocks of O
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = p.N;

  // ---- workgroup -> (head, query block) ----------------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  When the
  // head count allows, all query blocks of one head go to the same XCD so its
  // K/V stay in that XCD's L2; causal runs take the longest blocks first.
  const int nq = p.n_qblk;
  int bh, qb;
  {
    const int id = blockIdx.x;
    if (p.xcd_remap) {
      const int xcd = id & 7, slot = id >> 3;
      bh = xcd * (p.BH >> 3) + slot / nq;
      qb = slot % nq;
    } else {
      bh = id / nq;
      qb = id % nq;
    }
    if (CAUSAL) qb = nq - 1 - qb;
  }
  const int q0 = qb * BM;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ qh = p.q + head_off;
  const uint16_t* __restrict__ kh = p.k + head_off;
  const uint16_t* __restrict__ vh = p.v + head_off;
  const int wr0 = q0 + wave * 32 * QT;         // first query row of this wave

  // ---- Q fragments (B operand of S^T = K Q^T) ----------------------------
  // lane holds Q[row = lane % 32][8*(lane/32) + 16*kk .. +7]
  u32x4 qf[QT][DK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = min(wr0 + qt * 32 + (lane & 31), N - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 8 * (lane >> 5));
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      u32x4 x = src[2 * kk];
      if (p.q_mode == 1) x ^= 0x80008000u;     // negative scale: flip every sign
      if (p.q_mode == 2) x = (u32x4){0, 0, 0, 0};  // zero scale
      qf[qt][kk] = x;
    }
  }

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  // ---- K/V tile loads: HBM -> LDS directly ----------------------------------
  // One global_load_lds_dwordx4 moves 64 lanes x 16 bytes into 1 KiB of LDS,
  // lane l landing at base + 16*l.  LDS chunk index idx = row*CPR + slot, so
  // lane l of load t fetches the global chunk that the swizzle puts in that
  // slot.  Rows past the end repeat the last row: finite values whose scores
  // are masked, so they add exactly 0.
  auto issue_tile = [&](int j, int stage) {
    uint8_t* kdst = smem + stage * 2 * TILE_BYTES;
    uint8_t* vdst = kdst + TILE_BYTES;
#pragma unroll
    for (int t = 0; t < PER_W; ++t) {
      const int blk = wave * PER_W + t;            // 1 KiB block of the tile
      const int idx = blk * 64 + lane;             // LDS chunk index
      const int r = idx / CPR, slot = idx % CPR;
      const int grow = min(j * BC + r, N - 1);
      const uint16_t* krow = kh + (size_t)grow * D;
      const uint16_t* vrow = vh + (size_t)grow * D;
      __builtin_amdgcn_global_load_lds(krow + ((slot ^ (r & 7)) << 3),
                                       (__attribute__((address_space(3))) void*)(kdst + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vrow + ((slot ^ (2 * (r & 3))) << 3),
                                       (__attribute__((address_space(3))) void*)(vdst + blk * 1024), 16, 0, 0);
    }
  };

  // ---- running state -------------------------------------------------------
  const float c = p.c;                          // scale * log2(e), > 0
  float m[QT], l[QT];
  f32x16 oacc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.0f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qt][t][r] = 0.0f;
  }

  // per-lane constant parts of the LDS read addresses
  const int krow = lane & 31;                   // key row within a 32-key block
  const int kchunk = lane >> 5;                 // + 2*kk
  const int g = lane >> 4, gj = lane & 15;      // 16-lane group for the V reads
  const int vkey = 4 * (g >> 1) + (gj >> 2);    // + 32*kb + 16*h (and + 8)
  const int vcol = 16 * (g & 1) + 4 * (gj & 3); // + 32*t (head-dim column)

  issue_tile(0, 0);
  // raw-score margin before m moves (finite even for a tiny c)
  constexpr float RESCALE_LOG2 = BF16 ? 0.0f : 8.0f;
  const float thr = fminf(RESCALE_LOG2 / c, 3.0e38f);

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    // this wave's loads of tile j have landed; the barrier makes every
    // wave's loads visible and ends every wave's use of the other buffer
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(j + 1, stage ^ 1);
    const int c0 = j * BC;
    const uint8_t* kbase = smem + stage * 2 * TILE_BYTES;
    const uint8_t* vbase = kbase + TILE_BYTES;

    // a wave whose rows all precede this tile's first key has nothing to do
    if (!CAUSAL || c0 <= wr0 + 32 * QT - 1) {
      // ---- S^T = K Q^T --------------------------------------------------
      f32x16 s[QT][KB];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qt][kb][r] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 32 + krow;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
          const int ch = 2 * kk + kchunk;
          const u32x4 a = *reinterpret_cast<const u32x4*>(kbase + row * ROW_BYTES + ((ch ^ (row & 7)) << 4));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[qt][kb] = O::mfma(a, qf[qt][kk], s[qt][kb]);
        }
      }

      // ---- online softmax ------------------------------------------------
      u32x4 pb[QT][KB][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int r0 = wr0 + qt * 32;
        const int qrow = r0 + (lane & 31);
        const bool need_mask = (CAUSAL && c0 + BC - 1 > r0) || (c0 + BC > N);
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = c0 + kb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if ((CAUSAL && key > qrow) || key >= N) s[qt][kb][r] = -INFINITY;
            }
        }
        float mx = s[qt][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qt][kb][r]);
        mx = pair_max(mx);
        // move the reference only when some row outgrew it by the margin
        // (always on the first tile, where m is -inf)
        if (__builtin_amdgcn_ballot_w64(mx > m[qt] + thr) != 0) {
          const float mnew = fmaxf(m[qt], mx);
          // a row with no visible key yet keeps every factor finite
          const float mref = (mnew == -INFINITY) ? 0.0f : mnew;
          const float alpha = fast_exp2((m[qt] - mref) * c);   // 0 while m is -inf
          l[qt] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qt][t][r] *= alpha;
          m[qt] = mnew;
        }
        const float mc = ((m[qt] == -INFINITY) ? 0.0f : m[qt]) * c;
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(__builtin_fmaf(s[qt][kb][r], c, -mc));
            s[qt][kb][r] = pv;
            rs += pv;
          }
        l[qt] += rs;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pb[qt][kb][h][i] = O::pack(s[qt][kb][8 * h + 2 * i], s[qt][kb][8 * h + 2 * i + 1]);
      }

      // ---- O^T += V^T P^T ------------------------------------------------
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int col = 32 * t + vcol;
        const int chunk = col >> 3;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = kb * 32 + 16 * h + vkey;   // key & 3 == (key + 8) & 3
            const uint8_t* pa = vbase + key * ROW_BYTES + ((chunk ^ (2 * (key & 3))) << 4) + ((col & 7) << 1);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * ROW_BYTES));
            const u32x4 a = (u32x4){__builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]}),
                                    __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]}),
                                    __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){hi[0], hi[1]}),
                                    __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){hi[2], hi[3]})};
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) oacc[qt][t] = O::mfma(a, pb[qt][kb][h], oacc[qt][t]);
          }
      }
    }

  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m*c + log2 l) -----------------
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = pair_sum(l[qt]);
    const float inv = 1.0f / lt;
    const int qrow = wr0 + qt * 32 + (lane & 31);
    if (qrow < N) {
      float* orow = p.o + head_off + (size_t)qrow * D + 4 * (lane >> 5);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 val = {oacc[qt][t][4 * r4 + 0] * inv, oacc[qt][t][4 * r4 + 1] * inv,
                             oacc[qt][t][4 * r4 + 2] * inv, oacc[qt][t][4 * r4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * r4) = val;
        }
      if (lane < 32)
        p.lse[(size_t)bh * N + qrow] = (m[qt] * c + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
    }
  }
}

// ---- launch ------------------------------------------------------------------

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_one(const AttnParams& prm, int grid, hipStream_t stream) {
  constexpr int BC = 64, QT = 1, NW = 4;
  void* args[] = {const_cast<AttnParams*>(&prm)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<BF16, D, BC, QT, NW, CAUSAL>),
                         dim3(grid), dim3(NW * 64), args, 0, stream);
}

int block_rows(int d) {
  (void)d;
  return 4 * 32 * 1;
}

hipError_t launch_attn_fwd(bool bf16, int d, bool causal, AttnParams prm, hipStream_t stream) {
  const int bm = block_rows(d);
  prm.n_qblk = (prm.N + bm - 1) / bm;
  prm.xcd_remap = (prm.BH % 8 == 0) ? 1 : 0;
  const long long grid = (long long)prm.BH * prm.n_qblk;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int g = (int)grid;
  if (bf16) {
    if (d == 64) return causal ? launch_one<true, 64, true>(prm, g, stream) : launch_one<true, 64, false>(prm, g, stream);
    return causal ? launch_one<true, 128, true>(prm, g, stream) : launch_one<true, 128, false>(prm, g, stream);
  }
  if (d == 64) return causal ? launch_one<false, 64, true>(prm, g, stream) : launch_one<false, 64, false>(prm, g, stream);
  return causal ? launch_one<false, 128, true>(prm, g, stream) : launch_one<false, 128, false>(prm, g, stream);
}

}  // namespace ttc
