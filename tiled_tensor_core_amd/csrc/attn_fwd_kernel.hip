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
//   * workgroup = 4 waves; wave w owns 32 query rows, the workgroup 128 rows
//     of one (batch, head).  Two workgroups share a CU (<= 256 VGPRs per
//     wave, 64 KiB of LDS each), so every SIMD runs two waves.
//   * Q: each wave keeps its 32 rows in VGPRs for the whole pass, as the B
//     operand of v_mfma_f32_32x32x16 (8 consecutive head-dim elements per
//     lane), loaded once from HBM.
//   * K/V: 64-key tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no
//     VGPR staging).  The per-lane offsets are fixed for the whole pass; the
//     tile is selected by the scalar offset, so a tile costs no VALU address
//     arithmetic.  K and V each have two LDS buffers.
//   * software pipeline inside every wave, scheduled by hand: one tile is 32
//     steps (d = 128; 16 for d = 64), each one MFMA, the LDS reads of the
//     MFMA a few steps ahead, and a fixed slice of VALU work.  While the
//     MFMAs compute the scores of tile j+1, the VALU turns tile j's scores
//     into probabilities; while the MFMAs accumulate P_j V_j, the VALU
//     rescales O just ahead of them, sums the row and finds the maximum of
//     tile j+1.  A scheduling fence closes every step so the compiler keeps
//     this order; the K stream runs one tile ahead of the V stream and there
//     is one barrier per tile.
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
//   * tiles that need a mask (causal diagonal, keys past N) are the last
//     one or two of every workgroup; they run after the pipelined loop in a
//     plain loop that masks, and tiles wholly above a wave's rows are
//     skipped there (causal tile skipping).
//   * softmax in base 2: p = exp2(s*c - m*c) with c = scale*log2(e) folded
//     into one FMA; LSE = ln2 * (m*c + log2(l)) at the end.
//   * the running maximum m used as the exponent reference moves (and O, l
//     are rescaled by alpha = exp2((m_old - m_new)*c)) only when some row's
//     tile maximum exceeds it by more than a margin (in log2 units); else
//     alpha = 1.  bf16 uses a zero margin: m is the exact running maximum,
//     so a row's largest probability is exactly 1 and survives the bf16
//     rounding of P without error (this matters on peaky rows).  fp16, with
//     3 more bits of mantissa for P, keeps a stale reference until a row
//     outgrows it by 2^8 (p <= 256).  O / l and LSE do not depend on the
//     reference.
//
// LDS layout: K buffer 0, K buffer 1, V buffer 0, V buffer 1; each a [64][D]
// tile of bf16/fp16, rows of 2*D bytes split in 16-byte chunks.  The chunk
// index is XOR-swizzled per row so both read patterns hit all 64 banks once
// per phase:
//   D = 128: K chunk ^ (row & 15)         V chunk ^ 4*(row & 3)
//   D =  64: K chunk ^ ((row >> 1) & 7)   V chunk ^ 4*((row >> 1) & 1)
// (K is read 16 lanes x 16 bytes per phase, 16 consecutive rows at one
// chunk; V is read 32 lanes x 8 bytes per phase, 4 rows x two 32-byte
// column windows.)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_launch.h"

namespace ttc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

#define TTC_INLINE __device__ __attribute__((always_inline)) inline

// LDS pointer from a 32-bit LDS byte address
template <class T>
TTC_INLINE __attribute__((address_space(3))) T* lds_at(int a) {
  return (__attribute__((address_space(3))) T*)(size_t)(uint32_t)a;
}

// Element-type specific pieces: the 32x32x16 MFMA and the fp32 -> 16-bit
// pair conversion (round to nearest even) used for the probabilities.
template <bool BF16>
struct Ops;

template <>
struct Ops<true> {
  TTC_INLINE static f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  TTC_INLINE static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
};

template <>
struct Ops<false> {
  TTC_INLINE static f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  TTC_INLINE static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
};

// LDS swizzles (see the layout note above): the physical 16-byte chunk of
// logical chunk ch in key row r is ch ^ Swz::k(r) in a K tile and
// ch ^ Swz::v(r) in a V tile.
template <int D>
struct Swz;
template <>
struct Swz<128> {
  TTC_INLINE static int k(int r) { return r & 15; }
  TTC_INLINE static int v(int r) { return 4 * (r & 3); }
};
template <>
struct Swz<64> {
  TTC_INLINE static int k(int r) { return (r >> 1) & 7; }
  TTC_INLINE static int v(int r) { return 4 * ((r >> 1) & 1); }
};

// Row reductions across the two lane halves: lanes l and l ^ 32 hold the
// two halves of one query row.  v_permlane32_swap(x, x) gives lanes 0-31
// (own, lane + 32) and lanes 32-63 (lane - 32, own), so combining the two
// results yields the same value in both lanes.
TTC_INLINE float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
TTC_INLINE float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

TTC_INLINE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kBC = 64;        // keys per K/V tile
constexpr int kNW = 4;         // waves per workgroup
constexpr int kBM = kNW * 32;  // query rows per workgroup
constexpr int kLead = 3;       // LDS operand reads issued this many MFMAs ahead
constexpr int kChunks = 16;    // VALU slices per phase of a pipelined tile

// Per-wave state and the work of one key tile.
template <bool BF16, int D>
struct Wave {
  using O = Ops<BF16>;
  static constexpr int BC = kBC;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BC * ROW_BYTES;
  static constexpr int KB = BC / 32;         // 32-key blocks per tile
  static constexpr int DK = D / 16;          // k-steps of the score product
  static constexpr int DT = D / 32;          // 32-wide head-dim blocks of O
  static constexpr int NQK = DK * KB;        // score MFMAs per tile
  static constexpr int NPV = DT * KB * 2;    // P V MFMAs per tile
  static constexpr int NS = KB * 16;         // scores per lane per tile
  static_assert(NS == 32, "the VALU slicing below assumes 32 scores per lane");
  static_assert(kChunks % NQK == 0 || NQK % kChunks == 0, "slices must map onto steps");

  u32x4 qf[DK];      // Q rows (B operand of S^T = K Q^T)
  f32x16 oacc[DT];   // O^T accumulator of the wave's 32 rows
  u32x4 pb[KB][2];   // 16-bit P^T fragments (B operand of O^T += V^T P^T)
  float m, l;        // running maximum (raw score units) and row sum
  float c, thr;      // score multiplier |scale|*log2(e); margin before m moves
  float alpha;       // pending rescale factor of O and l for the current tile
  float mc;          // m * c, the exponent offset of the current tile
  bool moved;        // some row of the wave moved its reference maximum (alpha != 1)
  int kro[DK];       // LDS byte address of this lane's K operand (buffer 0)
  int vro[DT];       // LDS byte address of this lane's V^T operand (buffer 0)

  TTC_INLINE static float at(const f32x16 (&s)[KB], int v) { return s[v >> 4][v & 15]; }

  // ---- MFMA steps -------------------------------------------------------------
  // Score step i (kk = i / KB, kb = i % KB): S^T[kb] += K[kb-th 32 keys][kk] Q^T.
  TTC_INLINE u32x4 kop(int i, int kbuf) const {
    return *lds_at<u32x4>(kro[i / KB] + kbuf + (i % KB) * 32 * ROW_BYTES);
  }
  TTC_INLINE void qk(int i, u32x4 a, f32x16 (&s)[KB]) const {
    const int kk = i / KB, kb = i % KB;
    s[kb] = O::mfma(a, qf[kk], kk == 0 ? (f32x16){} : s[kb]);
  }
  // P V step i (t = i / (2 KB), kb = (i / 2) % KB, h = i % 2):
  // O^T[t] += V^T[t-th 32 dims][16 keys] P^T[16 keys].
  TTC_INLINE u32x4 vop(int i, int vbuf) const {
    const int t = i / (2 * KB), kb = (i / 2) % KB, h = i % 2;
    const int pa = vro[t] + vbuf + (kb * 32 + 16 * h) * ROW_BYTES;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(pa));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(pa + 8 * ROW_BYTES));
    return (u32x4){__builtin_bit_cast(uint32_t, (i16x2){lo[0], lo[1]}),
                   __builtin_bit_cast(uint32_t, (i16x2){lo[2], lo[3]}),
                   __builtin_bit_cast(uint32_t, (i16x2){hi[0], hi[1]}),
                   __builtin_bit_cast(uint32_t, (i16x2){hi[2], hi[3]})};
  }
  TTC_INLINE void pv(int i, u32x4 a) {
    const int t = i / (2 * KB), kb = (i / 2) % KB, h = i % 2;
    oacc[t] = O::mfma(a, pb[kb][h], oacc[t]);
  }

  // ---- softmax pieces ---------------------------------------------------------
  // Set the scores of keys a lane's row may not see to -inf.  The key of
  // s[kb][r] is c0 + kb*32 + 8*(r/4) + 4*(lane/32) + r%4; it is visible
  // when kb*32 + 8*(r/4) + r%4 <= lim.
  TTC_INLINE static void mask(f32x16 (&s)[KB], int lim) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
  // The row's tile maximum mx (both lane halves) moves the reference
  // maximum if some row of the wave outgrew it by the margin (always on the
  // first tile, where m is -inf); sets alpha and mc for the tile.
  TTC_INLINE void new_max(float mx) {
    mx = pair_max(mx);
    const bool move = __builtin_amdgcn_ballot_w64(mx > m + thr) != 0;
    moved = move;
    const float mnew = move ? fmaxf(m, mx) : m;
    // a row with no visible key yet keeps every factor finite
    const float mref = (mnew == -INFINITY) ? 0.0f : mnew;
    alpha = fast_exp2((m - mref) * c);  // 0 while m is -inf, 1 if m stays
    m = mnew;
    mc = mref * c;
  }
  TTC_INLINE void max_all(f32x16 (&s)[KB]) {
    float mx = s[0][0];
#pragma unroll
    for (int v = 1; v < NS; ++v) mx = fmaxf(mx, at(s, v));
    new_max(mx);
  }
  TTC_INLINE void prob(f32x16 (&s)[KB], int v) { s[v >> 4][v & 15] = fast_exp2(__builtin_fmaf(at(s, v), c, -mc)); }
  TTC_INLINE void pack(f32x16 (&s)[KB], int k) {  // k = (kb*2 + h)*4 + i
    const int kb = k >> 3, h = (k >> 2) & 1, i = k & 3;
    pb[kb][h][i] = O::pack(s[kb][8 * h + 2 * i], s[kb][8 * h + 2 * i + 1]);
  }
  TTC_INLINE void row_sum(f32x16 (&s)[KB]) {
    float t[NS / 2];
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) t[i] = at(s, 2 * i) + at(s, 2 * i + 1);
#pragma unroll
    for (int w = NS / 4; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) t[i] = t[i] + t[i + w];
    l = __builtin_fmaf(l, alpha, t[0]);
  }

  // ---- one tile without pipelining (masked tiles, short sequences) ----------
  TTC_INLINE void scores(f32x16 (&s)[KB], int kbuf) const {
#pragma unroll
    for (int i = 0; i < NQK; ++i) qk(i, kop(i, kbuf), s);
  }
  // O = alpha O + P V for the tile in s, whose maximum is already applied.
  TTC_INLINE void finish(f32x16 (&s)[KB], int vbuf) {
#pragma unroll
    for (int v = 0; v < NS; ++v) prob(s, v);
#pragma unroll
    for (int k = 0; k < 4 * KB * 2; ++k) pack(s, k);
    row_sum(s);
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
#pragma unroll
    for (int i = 0; i < NPV; ++i) pv(i, vop(i, vbuf));
  }

  // ---- one pipelined tile ------------------------------------------------------
  // On entry s holds tile j's scores with m, mc, alpha already set for it;
  // K buffer KBUF holds tile j+1's keys and V buffer VBUF tile j's values.
  // On exit sn holds tile j+1's scores, m/mc/alpha are set for tile j+1, and
  // O, l include tile j.
  //   phase 1 (NQK steps, MFMA: scores of tile j+1 into sn), VALU slices:
  //     0-7: p = exp2(s*c - mc) for 4 scores each; 8-11: 4 P^T packs each;
  //     12-15: 4 registers of O^T[0] *= alpha each
  //   phase 2 (NPV steps, MFMA: O^T[t] += V^T P^T, t-major), VALU slices:
  //     4(t-1)..4(t-1)+3: 4 registers of O^T[t] *= alpha each (t >= 1);
  //     0-7: first level of the row-sum tree (2 adds each); 8-11: second
  //     level; 12: third; 13: rest, l = alpha l + sum; 12-14: maximum tree
  //     of tile j+1; 15: new reference maximum, alpha, mc of tile j+1
  // RESCALE = false is the variant for tiles whose alpha is exactly 1.
  template <int KBUF, int VBUF, bool RESCALE>
  TTC_INLINE void pipe_tile(f32x16 (&s)[KB], f32x16 (&sn)[KB]) {
    constexpr int L = kLead, NSTEP = NQK + NPV;
    u32x4 op[L];
#pragma unroll
    for (int g = 0; g < L; ++g) op[g] = kop(g, KBUF);
    float rs[NS / 2];
    float mp[11], q[4];
#pragma unroll
    for (int g = 0; g < NSTEP; ++g) {
      const bool p1 = g < NQK;
      const int i = p1 ? g : g - NQK;
      const u32x4 a = op[g % L];
      if (g + L < NSTEP) op[g % L] = (g + L < NQK) ? kop(g + L, KBUF) : vop(g + L - NQK, VBUF);
      if (p1)
        qk(i, a, sn);
      else
        pv(i, a);
      const int n_steps = p1 ? NQK : NPV;
      const int c_lo = i * kChunks / n_steps, c_hi = (i + 1) * kChunks / n_steps;
#pragma unroll
      for (int cc = c_lo; cc < c_hi; ++cc) {
        if (p1) {
          if (cc < 8) {
#pragma unroll
            for (int v = 4 * cc; v < 4 * cc + 4; ++v) prob(s, v);
          } else if (cc < 12) {
#pragma unroll
            for (int k = 4 * (cc - 8); k < 4 * (cc - 8) + 4; ++k) pack(s, k);
          } else if (RESCALE) {
#pragma unroll
            for (int r = 4 * (cc - 12); r < 4 * (cc - 12) + 4; ++r) oacc[0][r] *= alpha;
          }
        } else {
          const int t = cc / 4 + 1;
          if (RESCALE && t < DT) {
#pragma unroll
            for (int r = 4 * (cc % 4); r < 4 * (cc % 4) + 4; ++r) oacc[t][r] *= alpha;
          }
          if (cc < 8) {
            rs[2 * cc] = at(s, 4 * cc) + at(s, 4 * cc + 1);
            rs[2 * cc + 1] = at(s, 4 * cc + 2) + at(s, 4 * cc + 3);
          } else if (cc < 12) {
            const int k = 2 * (cc - 8);
            rs[k] = rs[2 * k] + rs[2 * k + 1];
            rs[k + 1] = rs[2 * k + 2] + rs[2 * k + 3];
          } else if (cc == 12) {
#pragma unroll
            for (int k = 0; k < 4; ++k) rs[k] = rs[2 * k] + rs[2 * k + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              mp[k] = fmaxf(fmaxf(at(sn, 3 * k), at(sn, 3 * k + 1)), at(sn, 3 * k + 2));
          } else if (cc == 13) {
            rs[0] = (rs[0] + rs[1]) + (rs[2] + rs[3]);
            l = RESCALE ? __builtin_fmaf(l, alpha, rs[0]) : l + rs[0];
#pragma unroll
            for (int k = 4; k < 8; ++k)
              mp[k] = fmaxf(fmaxf(at(sn, 3 * k), at(sn, 3 * k + 1)), at(sn, 3 * k + 2));
          } else if (cc == 14) {
            mp[8] = fmaxf(fmaxf(at(sn, 24), at(sn, 25)), at(sn, 26));
            mp[9] = fmaxf(fmaxf(at(sn, 27), at(sn, 28)), at(sn, 29));
            mp[10] = fmaxf(at(sn, 30), at(sn, 31));
            q[0] = fmaxf(fmaxf(mp[0], mp[1]), mp[2]);
            q[1] = fmaxf(fmaxf(mp[3], mp[4]), mp[5]);
            q[2] = fmaxf(fmaxf(mp[6], mp[7]), mp[8]);
            q[3] = fmaxf(mp[9], mp[10]);
          } else {
            new_max(fmaxf(fmaxf(fmaxf(q[0], q[1]), q[2]), q[3]));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Start the loads of this wave's share of K or V tile j (rows j*BC ..) into
// LDS at dst: PER_W buffer_load_dwordx4 ... lds, lane offsets off[] within
// the tile.  Rows of the tile past N (only in the last tile) are clamped to
// row N-1, keeping the swizzled slot of the row they stand in for.
template <int PER_W, int ROW_BYTES, int BC>
TTC_INLINE void load_tile(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, const int* off, int j) {
#pragma unroll
  for (int t = 0; t < PER_W; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + t * 1024), 16, off[t], j * BC * ROW_BYTES, 0, 0);
}

template <bool BF16, int D, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64), amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(AttnParams p) {
  using W = Wave<BF16, D>;
  using S = Swz<D>;
  constexpr int BC = kBC, NW = kNW, BM = kBM;
  constexpr int KB = W::KB, DK = W::DK, DT = W::DT;
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = BC * ROW_BYTES;   // one K or V tile
  constexpr int PER_W = BC * CPR / 64 / NW;    // 1 KiB direct loads per wave per tile
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(4 * TILE_BYTES <= 65536, "LDS offsets must fit the instruction offset field");

  // K buffer 0 | K buffer 1 | V buffer 0 | V buffer 1
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];

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
  const int wr0 = q0 + wave * 32;              // first query row of this wave
  const int qrow = wr0 + (lane & 31);          // this lane's query row

  W w;
  // ---- Q fragments: lane holds Q[row = lane % 32][8*(lane/32) + 16*kk .. +7]
  {
    const int row = min(qrow, N - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + head_off + (size_t)row * D + 8 * (lane >> 5));
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      u32x4 x = src[2 * kk];
      if (p.q_mode == 1) x ^= 0x80008000u;         // negative scale: flip every sign
      if (p.q_mode == 2) x = (u32x4){0, 0, 0, 0};  // zero scale
      w.qf[kk] = x;
    }
  }

  // ---- K/V tile loads: HBM -> LDS directly ----------------------------------
  // One buffer_load_dwordx4 ... lds moves 64 lanes x 16 bytes into 1 KiB of
  // LDS, lane l landing at base + 16*l.  LDS chunk index idx = row*CPR + slot,
  // so lane l of load t fetches the global chunk that the swizzle puts in
  // that slot.  The buffer spans the head; the tile is the scalar offset.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head_off), 0, N * ROW_BYTES, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head_off), 0, N * ROW_BYTES, 0x00020000);
  const int first_idx = wave * PER_W * 64 + lane;   // LDS chunk index of this lane's first load
  int koff[PER_W], voff[PER_W];
#pragma unroll
  for (int t = 0; t < PER_W; ++t) {
    const int idx = first_idx + 64 * t;
    const int r = idx / CPR, slot = idx % CPR;
    koff[t] = r * ROW_BYTES + ((slot ^ S::k(r)) << 4);
    voff[t] = r * ROW_BYTES + ((slot ^ S::v(r)) << 4);
  }
  // The last tile's rows past N (if any) repeat row N-1 (finite values whose
  // scores are masked, so they add exactly 0), keeping the swizzled slot of
  // the row they stand in for.
  const int j_tail = (N - 1) / BC;
  auto tail_off = [&](const int (&off)[PER_W], int (&o)[PER_W]) {
#pragma unroll
    for (int t = 0; t < PER_W; ++t) {
      const int r = (first_idx + 64 * t) / CPR;
      o[t] = off[t] + (min(r, N - 1 - j_tail * BC) - r) * ROW_BYTES;
    }
  };
  uint8_t* const kdst = smem + wave * PER_W * 1024;                   // + buf * TILE_BYTES
  uint8_t* const vdst = smem + 2 * TILE_BYTES + wave * PER_W * 1024;  // + buf * TILE_BYTES
  auto load_k = [&](int j) {
    if (j == j_tail) {
      int o[PER_W];
      tail_off(koff, o);
      load_tile<PER_W, ROW_BYTES, BC>(krs, kdst + (j & 1) * TILE_BYTES, o, j);
    } else {
      load_tile<PER_W, ROW_BYTES, BC>(krs, kdst + (j & 1) * TILE_BYTES, koff, j);
    }
  };
  auto load_v = [&](int j) {
    if (j == j_tail) {
      int o[PER_W];
      tail_off(voff, o);
      load_tile<PER_W, ROW_BYTES, BC>(vrs, vdst + (j & 1) * TILE_BYTES, o, j);
    } else {
      load_tile<PER_W, ROW_BYTES, BC>(vrs, vdst + (j & 1) * TILE_BYTES, voff, j);
    }
  };

  // ---- per-lane LDS read addresses (buffer 0; buffer 1 is + TILE_BYTES) -------
  {
    const int lds0 = (int)(uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)smem;
    const int krow = lane & 31;                   // key row within a 32-key block
    const int kchunk = lane >> 5;                 // + 2*kk
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      w.kro[kk] = lds0 + krow * ROW_BYTES + (((2 * kk + kchunk) ^ S::k(krow)) << 4);
    const int g = lane >> 4, gj = lane & 15;      // 16-lane group for the V reads
    const int vkey = 4 * (g >> 1) + (gj >> 2);    // + 32*kb + 16*h (and + 8)
    const int vcol = 16 * (g & 1) + 4 * (gj & 3); // + 32*t (head-dim column)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int col = 32 * t + vcol;
      w.vro[t] = lds0 + 2 * TILE_BYTES + vkey * ROW_BYTES + (((col >> 3) ^ S::v(vkey)) << 4) + ((col & 7) << 1);
    }
  }

  // ---- running state -------------------------------------------------------
  w.c = p.c;                                    // |scale| * log2(e), > 0
  w.thr = p.thr;                                // raw-score margin before m moves
  w.m = -INFINITY;
  w.l = 0.0f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.oacc[t][r] = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  // mask limit of tile j for this lane (see Wave::mask), and whether any row
  // of this wave needs the mask there
  auto mask_lim = [&](int j) { return (CAUSAL ? min(qrow, N - 1) : N - 1) - j * BC - 4 * (lane >> 5); };
  auto needs_mask = [&](int j) { return (CAUSAL && j * BC + BC - 1 > wr0) || j * BC + BC > N; };
  // Tiles no row of the workgroup needs masked run software-pipelined: step j
  // handles tile j and computes tile j+1's scores and maximum, so both must
  // be such tiles; its loads (K_{j+2}, V_{j+1}) must not reach the tile that
  // ends past N.  The rest run in a plain loop.
  const int n_full = CAUSAL ? min(q0 / BC, N / BC) : N / BC;
  int n_pipe = max(0, min(n_full, n_tiles) - 1);
  if (n_tiles > N / BC) n_pipe = max(0, min(n_pipe, N / BC - 2));

  // Tile j's K sits in K buffer j%2 and its V in V buffer j%2.  Step j (with
  // the K stream one tile ahead): wait for K_{j+1}, V_j; start K_{j+2},
  // V_{j+1}; compute.  On entry to step j the scores of tile j are in sa
  // (masked) with the reference maximum, mc and alpha set for it.
  f32x16 sa[KB], sb[KB];
  load_k(0);
  load_v(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (1 < n_tiles) load_k(1);
  w.scores(sa, 0);
  if (needs_mask(0)) W::mask(sa, mask_lim(0));
  w.max_all(sa);

  auto top = [&](int j) {
    // K_{j+1} and V_j have landed for this wave; the barrier makes every
    // wave's loads visible and ends every wave's use of K_j and V_{j-1}
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < n_tiles) load_k(j + 2);
    if (j + 1 < n_tiles) load_v(j + 1);
  };
  auto top_full = [&](int j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < n_tiles) load_tile<PER_W, ROW_BYTES, BC>(krs, kdst + (j & 1) * TILE_BYTES, koff, j + 2);
    load_tile<PER_W, ROW_BYTES, BC>(vrs, vdst + ((j + 1) & 1) * TILE_BYTES, voff, j + 1);
  };
  // even tiles: K_{j+1} in buffer 1, V_j in buffer 0; odd tiles the other way
  int j = 0;
  for (; j + 1 < n_pipe; j += 2) {
    top_full(j);
    if (w.moved)
      w.template pipe_tile<TILE_BYTES, 0, true>(sa, sb);
    else
      w.template pipe_tile<TILE_BYTES, 0, false>(sa, sb);
    top_full(j + 1);
    if (w.moved)
      w.template pipe_tile<0, TILE_BYTES, true>(sb, sa);
    else
      w.template pipe_tile<0, TILE_BYTES, false>(sb, sa);
  }
  if (j < n_pipe) {
    top_full(j);
    w.template pipe_tile<TILE_BYTES, 0, true>(sa, sb);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sa[kb] = sb[kb];
    ++j;
  }

  // ---- remaining tiles (diagonal, tail), masked where needed ---------------------
  for (; j < n_tiles; ++j) {
    top(j);
    const int c0 = j * BC;
    // a wave whose rows all precede a tile's first key has nothing to do
    if (!CAUSAL || c0 <= wr0 + 31) w.finish(sa, (j & 1) * TILE_BYTES);
    if (j + 1 < n_tiles && (!CAUSAL || c0 + BC <= wr0 + 31)) {
      w.scores(sa, ((j + 1) & 1) * TILE_BYTES);
      if (needs_mask(j + 1)) W::mask(sa, mask_lim(j + 1));
      w.max_all(sa);
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m*c + log2 l) -----------------
  const float lt = pair_sum(w.l);
  const float inv = 1.0f / lt;
  if (qrow < N) {
    float* orow = p.o + head_off + (size_t)qrow * D + 4 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 val = {w.oacc[t][4 * r4 + 0] * inv, w.oacc[t][4 * r4 + 1] * inv,
                           w.oacc[t][4 * r4 + 2] * inv, w.oacc[t][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * r4) = val;
      }
    if (lane < 32)
      p.lse[(size_t)bh * N + qrow] = (w.m * w.c + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
  }
}

// ---- launch ------------------------------------------------------------------

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_one(const AttnParams& prm, int grid, hipStream_t stream) {
  void* args[] = {const_cast<AttnParams*>(&prm)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<BF16, D, CAUSAL>),
                         dim3(grid), dim3(kNW * 64), args, 0, stream);
}

int block_rows(int d) {
  (void)d;
  return kBM;
}

hipError_t launch_attn_fwd(bool bf16, int d, bool causal, AttnParams prm, hipStream_t stream) {
  const int bm = block_rows(d);
  prm.n_qblk = (prm.N + bm - 1) / bm;
  prm.xcd_remap = (prm.BH % 8 == 0) ? 1 : 0;
  // raw-score margin before the reference maximum moves: 0 for bf16 (exact
  // running maximum), 2^8 in probability units for fp16
  prm.thr = bf16 ? 0.0f : fminf(8.0f / prm.c, 3.0e38f);
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
