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
//   * an item is 128 query rows of one (batch, head); workgroup = 4 waves,
//     wave w owns 32 of the item's rows.  Two workgroups share a CU (<= 256
//     VGPRs per wave, 64 KiB of LDS each), so every SIMD runs two waves.
//     A second tile (NW = 8) takes 256 rows on 8 waves, one workgroup per
//     CU: each K/V tile in LDS then serves twice the rows.
//   * the kernel is persistent: the grid is as many workgroups as the chip
//     holds at once, each working through a fixed list of items (see the
//     item order in the kernel).  While an item's last tile is finished,
//     the next item's Q and first K/V tiles are already being loaded.
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
//     MFMAs compute the scores of tile j+1, the VALU turns most of tile j's
//     scores into probabilities; while the MFMAs accumulate P_j V_j, the
//     VALU finishes them, sums the row and (running-maximum mode) rescales O
//     just ahead of the MFMAs and finds the maximum of tile j+1.  A
//     scheduling fence closes every step so the compiler keeps this order;
//     the K stream runs one tile ahead of the V stream and there is one
//     barrier per tile.
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
//     one or two of every item; they run after the pipelined loop in a
//     loop that masks, and tiles wholly above a wave's rows are skipped
//     there (causal tile skipping).
//   * O leaves through LDS: each wave turns its accumulators row-major in
//     4 KiB of LDS so every store writes whole 128-byte row pieces.
//   * softmax in base 2: p = exp2(s*c - m*c) with c = scale*log2(e) folded
//     into one FMA; LSE = ln2 * (m*c + log2(l)) at the end.
//   * every row keeps two sums: l, of the unrounded fp32 p (for LSE), and
//     lo, of the 16-bit P the matrix cores multiply V by (v_dot2c against a
//     pair of ones, two P per instruction).  O = acc / lo is then a weighted
//     mean of the rows of V whose weights sum to 1, whatever the rounding of
//     P: dominant keys and keys tied at the maximum weigh the same in O's
//     numerator and denominator.  Neither O / lo nor LSE depends on the
//     exponent reference, so the reference need not be the running maximum:
//   * fixed-reference mode (the default): an item takes its first tile's row
//     maxima, raised by a headroom, as the reference for all its tiles, so
//     no later tile reduces a maximum or rescales O.  An item whose P leave
//     the range this allows is computed again with exact row maxima (rare:
//     a row must outgrow its first tile by 2^96 for bf16, 2^20 for fp16).
//   * running-maximum mode (the other variant): the reference m moves (and
//     O, l, lo are rescaled by alpha = exp2((m_old - m_new)*c)) when some
//     row's tile maximum exceeds it by more than a margin, 2^2 in
//     probability units for bf16 and 2^8 for fp16; else alpha = 1 and the
//     tile skips the 64 multiplies of O.
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

#include <algorithm>
#include <atomic>
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
typedef __attribute__((address_space(3))) uint8_t lds_u8;

#define TTC_INLINE __device__ __attribute__((always_inline)) inline

// LDS pointer from a 32-bit LDS byte address
template <class T>
TTC_INLINE __attribute__((address_space(3))) T* lds_at(int a) {
  return (__attribute__((address_space(3))) T*)(size_t)(uint32_t)a;
}

// Element-type specific pieces: the 32x32x16 MFMA, the fp32 -> 16-bit pair
// conversion (round to nearest even) used for the probabilities, and the sum
// of a packed pair.
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
  // acc + both 16-bit values of a packed pair (v_dot2c against ones)
  TTC_INLINE static float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
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
  TTC_INLINE static float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
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

// Maximum of three, NaN-propagating (v_maximum3_f32 on gfx950: no operand
// canonicalisation, unlike fmaxf in IEEE mode).
TTC_INLINE float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

constexpr int kBC = 64;        // keys per K/V tile
constexpr int kLead = 3;       // LDS operand reads issued this many MFMAs ahead
constexpr int kChunks = 16;    // VALU slices per phase of a pipelined tile
constexpr int kLoadEvery = 2;  // a pipelined tile issues one K/V tile load every this many steps

// Per-wave state and the work of one key tile.  FIXED: the wave runs in
// fixed-reference mode (see the kernel).
template <bool BF16, int D, bool FIXED>
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
  float m, l;        // running maximum (raw score units) and row sum of the fp32 p
  float lo;          // row sum of the 16-bit P that multiply V (O's normaliser)
  float c, thr;      // score multiplier |scale|*log2(e); margin before m moves
  float alpha;       // pending rescale factor of O and l for the current tile
  float mc;          // m * c, the exponent offset of the current tile
  bool moved;        // some row of the wave moved its reference maximum (alpha != 1)
  int kro[DK];       // byte offset of this lane's K operand in a K tile, per k-step
  int vro[DT];       // byte offset of this lane's V^T operand in a V tile, per d-block

  TTC_INLINE static float at(const f32x16 (&s)[KB], int v) { return s[v >> 4][v & 15]; }

  // ---- MFMA steps -------------------------------------------------------------
  // Score step i (kk = i / KB, kb = i % KB): S^T[kb] += K[kb-th 32 keys][kk] Q^T.
  TTC_INLINE u32x4 kop(int i, const lds_u8* kt) const {
    return *(const __attribute__((address_space(3))) u32x4*)(kt + kro[i / KB] + (i % KB) * 32 * ROW_BYTES);
  }
  TTC_INLINE void qk(int i, u32x4 a, f32x16 (&s)[KB]) const {
    const int kk = i / KB, kb = i % KB;
    s[kb] = O::mfma(a, qf[kk], kk == 0 ? (f32x16){} : s[kb]);
  }
  // P V step i (t = i / (2 KB), kb = (i / 2) % KB, h = i % 2):
  // O^T[t] += V^T[t-th 32 dims][16 keys] P^T[16 keys].  KBM: the steps run
  // key-block-major instead (kb = i / (2 DT), t = (i / 2) % DT), so the first
  // half of them needs only the first key block's P; every O^T[t] still
  // takes its four products in the same order.
  template <bool KBM = false>
  TTC_INLINE u32x4 vop(int i, const lds_u8* vt) const {
    const int t = KBM ? (i / 2) % DT : i / (2 * KB), kb = KBM ? i / (2 * DT) : (i / 2) % KB, h = i % 2;
    const lds_u8* pa = vt + vro[t] + (kb * 32 + 16 * h) * ROW_BYTES;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * ROW_BYTES));
    return (u32x4){__builtin_bit_cast(uint32_t, (i16x2){lo[0], lo[1]}),
                   __builtin_bit_cast(uint32_t, (i16x2){lo[2], lo[3]}),
                   __builtin_bit_cast(uint32_t, (i16x2){hi[0], hi[1]}),
                   __builtin_bit_cast(uint32_t, (i16x2){hi[2], hi[3]})};
  }
  template <bool KBM = false>
  TTC_INLINE void pv(int i, u32x4 a) {
    const int t = KBM ? (i / 2) % DT : i / (2 * KB), kb = KBM ? i / (2 * DT) : (i / 2) % KB, h = i % 2;
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
  // The causal mask of a tile that starts delta = c0 - wr0 keys after the
  // wave's first query row, for a tile wholly inside the sequence.  Score
  // e = 16 kb + r of a lane holds key c0 + 32 kb + 8 (r/4) + r%4 + 4 (lane/32)
  // for query row wr0 + lane % 32; the key is hidden when it follows the row,
  // that is when rel + 32 kb + 8 (r/4) + r%4 > 0 with the per-lane
  // rel = delta + 4 (lane/32) - lane % 32: one compare with a constant and
  // one select per score, and no branch (keys past N follow every row below
  // N, so this mask hides them as well).
  TTC_INLINE static int diag_rel(int delta) {
    const int ln = __lane_id();
    return delta + 4 * (ln >> 5) - (ln & 31);
  }
  TTC_INLINE static void diag_mask_one(f32x16 (&s)[KB], int rel, int e) {
    const int kb = e >> 4, r = e & 15;
    s[kb][r] = (rel > -(32 * kb + 8 * (r >> 2) + (r & 3))) ? -INFINITY : s[kb][r];
  }
  TTC_INLINE static void diag_mask(f32x16 (&s)[KB], int delta) {
    const int rel = diag_rel(delta);
#pragma unroll
    for (int e = 0; e < NS; ++e) diag_mask_one(s, rel, e);
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
    for (int v = 1; v < NS; ++v) mx = __builtin_elementwise_maximum(mx, at(s, v));
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
    // the same for the packed 16-bit P (after pack()): four chains of four
    float r4[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      r4[c4] = O::sum2(pb[c4 >> 1][c4 & 1][0], 0.0f);
#pragma unroll
      for (int i = 1; i < 4; ++i) r4[c4] = O::sum2(pb[c4 >> 1][c4 & 1][i], r4[c4]);
    }
    lo = __builtin_fmaf(lo, alpha, (r4[0] + r4[1]) + (r4[2] + r4[3]));
  }

  // ---- one tile without pipelining (masked tiles, short sequences) ----------
  TTC_INLINE void scores(f32x16 (&s)[KB], const lds_u8* kt) const {
#pragma unroll
    for (int i = 0; i < NQK; ++i) qk(i, kop(i, kt), s);
  }
  // O = alpha O + P V for the tile in s, whose maximum is already applied.
  TTC_INLINE void finish(f32x16 (&s)[KB], const lds_u8* vt) {
#pragma unroll
    for (int v = 0; v < NS; ++v) prob(s, v);
#pragma unroll
    for (int k = 0; k < 4 * KB * 2; ++k) pack(s, k);
    row_sum(s);
    if (moved) {   // wave-uniform: alpha is exactly 1 otherwise
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) pv(i, vop(i, vt));
  }

  // ---- one pipelined tile ------------------------------------------------------
  // On entry s holds tile j's scores with m, mc, alpha already set for it;
  // kt holds tile j+1's keys and vt tile j's values.
  // On exit sn holds tile j+1's scores, m/mc/alpha are set for tile j+1, and
  // O, l include tile j.
  //   phase 1 (NQK steps, MFMA: scores of tile j+1 into sn), VALU slices:
  //     0-7: p = exp2(s*c - mc) for 4 scores each; 8-11: 4 P^T packs each;
  //     12-15: 4 registers of O^T[0] *= alpha each
  //   phase 2 (NPV steps, MFMA: O^T[t] += V^T P^T, t-major), VALU slices:
  //     4(t-1)..4(t-1)+3: 4 registers of O^T[t] *= alpha each (t >= 1);
  //     0-7: first level of the row-sum tree (2 adds each) and two pair
  //     sums of the packed P each; 8-11: second level; 12: third; 13: rest,
  //     l = alpha l + sum, lo = alpha lo + packed sum; 12-14: maximum tree
  //     of tile j+1; 15: new reference maximum, alpha, mc of tile j+1
  // RESCALE = false is the variant for tiles whose alpha is exactly 1.
  // ld(k), k = 0 .. NLOAD-1, issues this wave's k-th load of the tiles the
  // step prefetches; the loads are spread over the first steps so their LDS
  // writes do not all land with the tile's first reads.
  // MAXN = false leaves tile j+1's maximum (and m, mc, alpha) to the caller,
  // for a next tile that must be masked first.
  // MASKN: tile j+1 is a causal diagonal tile starting mdelta keys after
  // the wave's first row; its mask goes in during slices 8-11 of phase 2,
  // ahead of the maximum.
  template <bool RESCALE, int NLOAD, class LD, bool MAXN = true, bool MASKN = false>
  TTC_INLINE void pipe_tile(f32x16 (&s)[KB], f32x16 (&sn)[KB], const lds_u8* kt, const lds_u8* vt,
                            const LD& ld, int mdelta = 0) {
    constexpr int L = kLead, NSTEP = NQK + NPV;
    u32x4 op[L];
#pragma unroll
    for (int g = 0; g < L; ++g) op[g] = kop(g, kt);
    float rs[NS / 2], ro[4];
    float mp[10], q[4];
    int mrel = 0;   // MASKN: the per-lane offset of diag_rel
#pragma unroll
    for (int g = 0; g < NSTEP; ++g) {
      const bool p1 = g < NQK;
      const int i = p1 ? g : g - NQK;
      const u32x4 a = op[g % L];
      if (g + L < NSTEP) op[g % L] = (g + L < NQK) ? kop(g + L, kt) : vop(g + L - NQK, vt);
      if (p1)
        qk(i, a, sn);
      else
        pv(i, a);
      if (g % kLoadEvery == 0 && g / kLoadEvery < NLOAD) ld(g / kLoadEvery);
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
          if (MASKN && cc >= 8 && cc < 12) {
            if (cc == 8) mrel = diag_rel(mdelta);
#pragma unroll
            for (int e = 8 * (cc - 8); e < 8 * (cc - 8) + 8; ++e) diag_mask_one(sn, mrel, e);
          }
          if (RESCALE && t < DT) {
#pragma unroll
            for (int r = 4 * (cc % 4); r < 4 * (cc % 4) + 4; ++r) oacc[t][r] *= alpha;
          }
          if (cc < 8) {
            rs[2 * cc] = at(s, 4 * cc) + at(s, 4 * cc + 1);
            rs[2 * cc + 1] = at(s, 4 * cc + 2) + at(s, 4 * cc + 3);
            // the packed P of slice cc: dwords 2cc, 2cc+1 of chain cc/2
            const int c4 = cc >> 1, i0 = 2 * (cc & 1);
            ro[c4] = O::sum2(pb[c4 >> 1][c4 & 1][i0], (cc & 1) ? ro[c4] : 0.0f);
            ro[c4] = O::sum2(pb[c4 >> 1][c4 & 1][i0 + 1], ro[c4]);
          } else if (cc < 12) {
            const int k = 2 * (cc - 8);
            rs[k] = rs[2 * k] + rs[2 * k + 1];
            rs[k + 1] = rs[2 * k + 2] + rs[2 * k + 3];
          } else if (cc == 12) {
#pragma unroll
            for (int k = 0; k < 4; ++k) rs[k] = rs[2 * k] + rs[2 * k + 1];
            ro[0] = ro[0] + ro[1];
            ro[2] = ro[2] + ro[3];
            if (MAXN) {
#pragma unroll
              for (int k = 0; k < 4; ++k) mp[k] = max3(at(sn, 3 * k), at(sn, 3 * k + 1), at(sn, 3 * k + 2));
            }
          } else if (cc == 13) {
            rs[0] = (rs[0] + rs[1]) + (rs[2] + rs[3]);
            l = RESCALE ? __builtin_fmaf(l, alpha, rs[0]) : l + rs[0];
            lo = RESCALE ? __builtin_fmaf(lo, alpha, ro[0] + ro[2]) : lo + (ro[0] + ro[2]);
            if (MAXN) {
#pragma unroll
              for (int k = 4; k < 8; ++k) mp[k] = max3(at(sn, 3 * k), at(sn, 3 * k + 1), at(sn, 3 * k + 2));
            }
          } else if (!MAXN) {
          } else if (cc == 14) {
            mp[8] = max3(at(sn, 24), at(sn, 25), at(sn, 26));
            mp[9] = max3(at(sn, 27), at(sn, 28), at(sn, 29));
            q[0] = max3(mp[0], mp[1], mp[2]);
            q[1] = max3(mp[3], mp[4], mp[5]);
            q[2] = max3(mp[6], mp[7], mp[8]);
            q[3] = max3(mp[9], at(sn, 30), at(sn, 31));
          } else {
            new_max(max3(q[0], q[1], __builtin_elementwise_maximum(q[2], q[3])));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- one pipelined tile with a fixed exponent reference ---------------------
  // The step of fixed-reference mode: as pipe_tile, but no maximum, no
  // rescale, and a schedule that spreads the VALU work evenly over the two
  // phases (an exponential costs twice an FMA, so a phase doing all 32
  // would carry most of the step's VALU time) and keeps running sums instead
  // of a reduction tree.  The P V steps run key-block-major, so the second
  // key block's P is needed only halfway through phase 2:
  //   phase 1 (scores of tile j+1): p = exp2(s*c - mc) of scores 0-23, two
  //     and one in alternate slices; each pair packed a slice after it
  //   phase 2 (O^T += V^T P^T), slices 0-7: p of scores 24-31, one a slice,
  //     and the packs of scores 22-29; slice 8: the pack of scores 30, 31
  //     (read by the P V step after it); slices 8-15: all 32 p into four
  //     chains of l; every slice: packed dword cc into the chain of lo; at
  //     cc = 15 the sums join l and lo.  MASKN: the causal mask of tile j+1
  //     in slices 8-11, as in pipe_tile.
  template <int NLOAD, class LD, bool MASKN = false>
  TTC_INLINE void pipe_tile_fixed(f32x16 (&s)[KB], f32x16 (&sn)[KB], const lds_u8* kt, const lds_u8* vt,
                                  const LD& ld, int mdelta = 0) {
    constexpr int L = kLead, NSTEP = NQK + NPV;
    static_assert(kChunks == 16 && NS == 32, "two scores and one packed dword per slice");
    u32x4 op[L];
#pragma unroll
    for (int g = 0; g < L; ++g) op[g] = kop(g, kt);
    float ra = 0.0f, rb = 0.0f, rc = 0.0f, rd = 0.0f, rp = 0.0f;
    int mrel = 0;   // MASKN: the per-lane offset of diag_rel
    // probabilities done after phase-1 slice cc: 2, 3, 5, 6, ..., 24
    auto done1 = [](int cc) { return cc < 0 ? 0 : (3 * (cc + 1) + 1) / 2; };
#pragma unroll
    for (int g = 0; g < NSTEP; ++g) {
      const bool p1 = g < NQK;
      const int i = p1 ? g : g - NQK;
      const u32x4 a = op[g % L];
      if (g + L < NSTEP) op[g % L] = (g + L < NQK) ? kop(g + L, kt) : vop<true>(g + L - NQK, vt);
      if (p1)
        qk(i, a, sn);
      else
        pv<true>(i, a);
      if (g % kLoadEvery == 0 && g / kLoadEvery < NLOAD) ld(g / kLoadEvery);
      const int n_steps = p1 ? NQK : NPV;
      const int c_lo = i * kChunks / n_steps, c_hi = (i + 1) * kChunks / n_steps;
#pragma unroll
      for (int cc = c_lo; cc < c_hi; ++cc) {
        if (p1) {
          // probabilities 0-23, one or two a slice; each pack a slice after its pair
#pragma unroll
          for (int v = done1(cc - 1); v < done1(cc); ++v) prob(s, v);
#pragma unroll
          for (int k = done1(cc - 2) / 2; k < done1(cc - 1) / 2; ++k) pack(s, k);
        } else {
          // slices 0-7 (the first key block's P V): probabilities 24-31,
          // packs 11-14 and the packed sum of key block 0; slices 8-15: the
          // sums of all 32 probabilities, pack 15, the packed sum of key block 1
          if (cc < 8) {
            prob(s, 24 + cc);
            if (cc == 0) pack(s, 11);
            if (cc >= 2 && (cc & 1) == 0) pack(s, 11 + cc / 2);
          } else if (cc == 8) {
            pack(s, 15);
          }
          if (MASKN && cc >= 8 && cc < 12) {
            if (cc == 8) mrel = diag_rel(mdelta);
#pragma unroll
            for (int e = 8 * (cc - 8); e < 8 * (cc - 8) + 8; ++e) diag_mask_one(sn, mrel, e);
          }
          if (cc >= 8) {
            const int v0 = 4 * (cc - 8);
            ra = cc == 8 ? at(s, v0) : ra + at(s, v0);
            rb = cc == 8 ? at(s, v0 + 1) : rb + at(s, v0 + 1);
            rc = cc == 8 ? at(s, v0 + 2) : rc + at(s, v0 + 2);
            rd = cc == 8 ? at(s, v0 + 3) : rd + at(s, v0 + 3);
          }
          rp = O::sum2(pb[cc >> 3][(cc >> 2) & 1][cc & 3], rp);
          if (cc == 15) {
            l += (ra + rb) + (rc + rd);
            lo += rp;
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
//
// The load is issued from inline assembly, so the compiler does not see it as
// a write of LDS.  Seen as one, it makes every later LDS read that it cannot
// prove to be in another buffer (a buffer chosen at run time, or one of more
// distinct load sites than it tracks) wait until all loads in flight have
// landed -- in the middle of a tile, a full memory round trip.  Every tile a
// load fills is read only after the wait at the start of a later step
// (vmcnt(0), then a workgroup barrier), so no other wait is needed.  The
// buffer resource is a plain 4-dword descriptor in scalar registers; M0 holds
// the LDS address, and one wait state separates its write from the load.
TTC_INLINE void load_one(u32x4 rs, lds_u8* dst, int off, int soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
  // the scalar offset must be an SGPR: a compile-time constant would
  // otherwise be printed as a literal, which the instruction cannot take
  // (soff is uniform by construction; readfirstlane states it where the
  // compiler cannot prove it)
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("" : "+s"(soff));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}


// The same descriptor as head_rsrc below, as four dwords: base address
// (48 bits, stride 0), size in bytes, and the format word.
TTC_INLINE u32x4 load_rsrc(const void* base, unsigned nbytes) {
  const uint64_t a = (uint64_t)(size_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nbytes, 0x00020000u};
}

// Buffer resource spanning nbytes from base (one head's K, V or O); loads
// outside it return 0, stores outside it are dropped.
TTC_INLINE __amdgpu_buffer_rsrc_t head_rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

// Stores of O are marked non-temporal (cache policy bit 1, "nt" on gfx950):
// O is written once, and keeping it out of L2 leaves room for the K/V tiles
// the other query blocks of a head still read.
TTC_INLINE void store_b128(__amdgpu_buffer_rsrc_t rs, f32x4 v, unsigned voff) {
  // the hardware reads the 32-bit offset as unsigned
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)voff, 0, 2);
}

// NW waves per workgroup, 32 query rows each: NW = 4 (128-row items, two
// workgroups per compute unit) or 8 (256-row items, one workgroup per
// compute unit, each K/V tile shared by twice the rows).
template <bool BF16, int D, bool CAUSAL, bool FIXED, int NW>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(AttnParams p) {
  using W = Wave<BF16, D, FIXED>;
  using S = Swz<D>;
  constexpr int BC = kBC, BM = NW * 32;
  constexpr int KB = W::KB, DK = W::DK, DT = W::DT;
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = BC * ROW_BYTES;   // one K or V tile
  constexpr int PER_W = BC * CPR / 64 / NW;    // 1 KiB direct loads per wave per tile
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(4 * TILE_BYTES <= 65536, "LDS offsets must fit the instruction offset field");

  // two K and two V tile buffers, each its own LDS object: the compiler can
  // then tell that a direct-to-LDS load into one buffer does not touch the
  // buffer being read, and need not wait for the load before reading
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE_BYTES];
  lds_u8* const K0 = (lds_u8*)k_lds0;
  lds_u8* const K1 = (lds_u8*)k_lds1;
  lds_u8* const V0 = (lds_u8*)v_lds0;
  lds_u8* const V1 = (lds_u8*)v_lds1;
  // d = 64: a separate 16 KiB for turning O row-major before it is stored
  // (d = 128 uses the V buffer the last tile read; see the epilogue)
  // (8 waves need 32 KiB, more than a V buffer, for either head dim)
  constexpr bool OWN_STAGE = D == 64 || NW != 4;
  constexpr int STAGE_BYTES = OWN_STAGE ? NW * 4096 : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t o_lds[STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = p.N;
  const unsigned HEAD_BYTES = (unsigned)N * ROW_BYTES;

  // ---- work items ------------------------------------------------------------
  // An item is one (head, query block).  The grid holds only as many
  // workgroups as the chip runs at once, and each one works through a fixed
  // list of items, so no workgroup waits to be dispatched and the last wave
  // of work is not left to chance.  Workgroups are dispatched round-robin
  // over the 8 XCDs (id % 8); when the head count allows, the heads are split
  // into 8 equal domains, one per XCD, so a head's K/V stay in one L2.  A
  // domain's items are listed group by group (gh heads per group), longest
  // first within a group (causal blocks further down the sequence see more
  // keys), and dealt out in rounds of one item per workgroup, the direction
  // of the deal alternating between rounds: over two rounds each workgroup
  // gets a long item and a short one whose costs add up to about the same.
  const int nq = p.n_qblk;
  const int dom = p.n_dom == 8 ? (int)(blockIdx.x & 7) : 0;
  const int wk = p.n_dom == 8 ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int nw = p.n_work, hd = p.BH / p.n_dom, gh = p.grp;
  const int dom_items = hd * nq;
  auto item = [&](int t, int& bh, int& qb) {
    const int pos = t * nw + ((t & 1) ? nw - 1 - wk : wk);
    if (pos >= dom_items) return false;
    const int g = pos / (gh * nq), k = pos - g * (gh * nq);
    const int gs = min(gh, hd - g * gh);   // heads in this group
    const int r = k / gs;
    bh = dom * hd + g * gh + (k - r * gs);
    qb = CAUSAL ? nq - 1 - r : r;
    return true;
  };
  auto tiles_of = [&](int qb) { return ((CAUSAL ? min(N, qb * BM + BM) : N) + BC - 1) / BC; };

  W w;
  // ---- Q fragments: lane holds Q[row = lane % 32][8*(lane/32) + 16*kk .. +7].
  // Plain loads into the fragment registers; the sign fix for a negative or
  // zero scale is applied once they have landed.
  auto load_q = [&](int bh, int qb) {
    const int row = min(qb * BM + wave * 32 + (lane & 31), N - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + (size_t)bh * N * D + (size_t)row * D + 8 * (lane >> 5));
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) w.qf[kk] = __builtin_nontemporal_load(src + 2 * kk);   // read once
  };

  // ---- K/V tile loads: HBM -> LDS directly ----------------------------------
  // One buffer_load_dwordx4 ... lds moves 64 lanes x 16 bytes into 1 KiB of
  // LDS, lane l landing at base + 16*l.  LDS chunk index idx = row*CPR + slot,
  // so lane l of load t fetches the global chunk that the swizzle puts in
  // that slot.  The buffer spans the head; the tile is the scalar offset.
  // The per-lane offsets depend on the lane only.  They are recomputed at
  // the start of every item (from a lane number the compiler cannot see
  // through) rather than kept live across items, where they would only take
  // up registers in the epilogue.
  // A wave's load t of a tile covers the rows 64t/CPR after those of its
  // load 0.  The V swizzle depends only on row bits those rows share, so V
  // load t fetches at the lane offset of load 0 plus 1 KiB * t; the K swizzle
  // adds 4t to the swizzle index (both head dims), so K load t fetches at
  // (lane offset of load 0) ^ 64t, plus 1 KiB * t.  The 1 KiB * t goes into
  // the scalar offset: one VGPR for all V loads, one per K load.
  const int first_idx = wave * PER_W * 64 + lane;   // LDS chunk index of this lane's first load
  auto lane_offsets = [&](int ln, int& ko, int& vo) {
    const int idx = wave * PER_W * 64 + ln;
    const int r = idx / CPR, slot = idx % CPR;
    ko = r * ROW_BYTES + ((slot ^ S::k(r)) << 4);
    vo = r * ROW_BYTES + ((slot ^ S::v(r)) << 4);
  };
  int koff, voff;
  lane_offsets(lane, koff, voff);
  // lane offset of K load t, kept for the whole item (four VGPRs instead of
  // an XOR per load)
  int kofs[PER_W];
  auto set_kofs = [&]() {
#pragma unroll
    for (int t = 0; t < PER_W; ++t) kofs[t] = koff ^ (64 * t);
  };
  set_kofs();
  auto koff_t = [&](int t) { return kofs[t]; };
  // The last tile's rows past N (if any) repeat row N-1 (finite values whose
  // scores are masked, so they add exactly 0), keeping the swizzled slot of
  // the row they stand in for.
  const int j_tail = (N - 1) / BC;
  auto tail_delta = [&](int t) {
    // recomputed where used: kept live, these would only take up registers
    int fi = first_idx;
    asm volatile("" : "+v"(fi));
    const int r = (fi + 64 * t) / CPR;
    return (min(r, N - 1 - j_tail * BC) - r) * ROW_BYTES;
  };
  const int wofs = wave * PER_W * 1024;   // this wave's share of a tile
  // K tile j
  auto load_k = [&](u32x4 rs, lds_u8* buf, int j) {
#pragma unroll
    for (int t = 0; t < PER_W; ++t)
      load_one(rs, buf + wofs + t * 1024, koff_t(t) + (j == j_tail ? tail_delta(t) : 0), j * TILE_BYTES + t * 1024);
  };
  // V tile j: load t at lane offset vo + 1 KiB * t (scalar part)
  auto load_v = [&](u32x4 rs, int vo, lds_u8* buf, int j) {
#pragma unroll
    for (int t = 0; t < PER_W; ++t)
      load_one(rs, buf + wofs + t * 1024, vo + (j == j_tail ? tail_delta(t) : 0), j * TILE_BYTES + t * 1024);
  };

  // ---- per-lane LDS read offsets within a tile ------------------------------------
  auto read_offsets = [&](int ln) {
    const int krow = ln & 31;                     // key row within a 32-key block
    const int kchunk = ln >> 5;                   // + 2*kk
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      w.kro[kk] = krow * ROW_BYTES + (((2 * kk + kchunk) ^ S::k(krow)) << 4);
    const int g = ln >> 4, gj = ln & 15;          // 16-lane group for the V reads
    const int vkey = 4 * (g >> 1) + (gj >> 2);    // + 32*kb + 16*h (and + 8)
    const int vcol = 16 * (g & 1) + 4 * (gj & 3); // + 32*t (head-dim column)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int col = 32 * t + vcol;
      w.vro[t] = vkey * ROW_BYTES + (((col >> 3) ^ S::v(vkey)) << 4) + ((col & 7) << 1);
    }
  };
  w.c = p.c;                                    // |scale| * log2(e), > 0
  w.thr = p.thr;                                // raw-score margin before m moves

  auto wait_all = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // ---- the first item's operands ------------------------------------------------
  // Tile j's K sits in K buffer j%2 and its V in V buffer j%2.  An item
  // starts with its Q, K_0, K_1 and V_0 in flight; the previous item issued
  // them at its last tile (V_0 only when V buffer 0 was free then).
  // Of the two workgroups on a CU the older one wins issue arbitration, and
  // with equal lists it would finish well before the younger one.  Each
  // workgroup therefore lowers its priority as it gets through its list
  // (3 for the first half of its tiles, 2 to three quarters, 1 to nine
  // tenths, then 0): whichever of the two is behind wins, and they finish
  // together.
  int tot_tiles = 0;
  for (int t = 0;; ++t) {
    int b2, q2;
    if (!item(t, b2, q2)) break;
    tot_tiles += tiles_of(q2);
  }
  // with the priority scheme off every threshold is 0: the priority stays 0
  const int th1 = p.prio ? tot_tiles / 2 : 0, th2 = p.prio ? (3 * tot_tiles) / 4 : 0,
            th3 = p.prio ? (9 * tot_tiles) / 10 : 0;
  int done_tiles = 0;
  auto progress = [&](int n) {
    done_tiles += n;
    if (done_tiles < th1)
      __builtin_amdgcn_s_setprio(3);
    else if (done_tiles < th2)
      __builtin_amdgcn_s_setprio(2);
    else if (done_tiles < th3)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  };
  int t_item = 0, bh, qb;
  if (!item(0, bh, qb)) return;
  u32x4 krs = load_rsrc(p.k + (size_t)bh * N * D, HEAD_BYTES);
  u32x4 vrs = load_rsrc(p.v + (size_t)bh * N * D, HEAD_BYTES);
  int n_tiles = tiles_of(qb);
  load_q(bh, qb);
  load_k(krs, K0, 0);
  load_v(vrs, voff, V0, 0);
  if (1 < n_tiles) load_k(krs, K1, 1);
  bool v0_late = false;
  f32x16 sa[KB], sb[KB];
  // Fixed-reference mode (FIXED): an item keeps the maximum of its first
  // tile (raised by p.headroom log2 units) as each row's exponent reference
  // throughout, so no later tile needs its maximum or a rescale of O.  O / lo is exact whatever the
  // reference; only the range of P depends on it.  Every P, and every P V
  // sum, stays finite while the row sums lo do (fp16: lo finite; bf16: lo at
  // most p.l_max = 2^48, which also leaves P V sums far from overflow).  A
  // wave whose lo does not (or is NaN) leaves item index + 1 in redo_tag,
  // and the workgroup computes that item again with each row's exact
  // maximum as its reference (found by a pass over the item's K tiles
  // first), so every p <= 1; the item's O and LSE are overwritten.  The tag
  // is read after the barrier that starts the next item (after the last
  // item, after one more barrier), and written only in an epilogue, at
  // least one barrier later.
  __shared__ int redo_tag;
  if (FIXED && threadIdx.x == 0) redo_tag = -1;
  int redone = -1;     // the tag of the last item computed again

  for (;;) {
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      lane_offsets(ln, koff, voff);
      set_kofs();
      read_offsets(ln);
    }
    // the item's loads have landed, and every wave is done with the previous
    // item's buffers
    wait_all();
    bool exact = false;   // this item is computed again, with exact row maxima
    if constexpr (FIXED) {
      const int tag = __builtin_amdgcn_readfirstlane(redo_tag);
      if (tag == t_item && tag != redone) {
        // the previous item's P left the fixed reference's range: load its
        // operands again (over the next item's, which are loaded again later)
        redone = tag;
        --t_item;
        item(t_item, bh, qb);
        krs = load_rsrc(p.k + (size_t)bh * N * D, HEAD_BYTES);
        vrs = load_rsrc(p.v + (size_t)bh * N * D, HEAD_BYTES);
        n_tiles = tiles_of(qb);
        load_q(bh, qb);
        load_k(krs, K0, 0);
        load_v(vrs, voff, V0, 0);
        if (1 < n_tiles) load_k(krs, K1, 1);
        v0_late = false;
        wait_all();
        exact = true;
      }
    }
    if (v0_late) load_v(vrs, voff, V0, 0);
    if (p.q_mode != 0) {
#pragma unroll
      for (int kk = 0; kk < DK; ++kk)   // negative scale: flip every sign; zero scale: zero
        w.qf[kk] = p.q_mode == 1 ? (w.qf[kk] ^ 0x80008000u) : (u32x4){0, 0, 0, 0};
    }
    const int q0 = qb * BM;
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const int wr0 = q0 + wave * 32;              // first query row of this wave
    const int qrow = wr0 + (lane & 31);          // this lane's query row

    // mask limit of tile j for this lane (see Wave::mask), and whether any row
    // of this wave needs the mask there
    auto mask_lim = [&](int j) { return (CAUSAL ? min(qrow, N - 1) : N - 1) - j * BC - 4 * (lane >> 5); };
    auto needs_mask = [&](int j) { return (CAUSAL && j * BC + BC - 1 > wr0) || j * BC + BC > N; };
    auto apply_mask = [&](f32x16 (&s)[KB], int j) {
      if (!needs_mask(j)) return;
      if (CAUSAL)   // keys past N follow every row below N
        W::diag_mask(s, j * BC - wr0);
      else
        W::mask(s, mask_lim(j));
    };

    // ---- exact row maxima of an item computed again (rare) -------------------
    // The item's K tiles stream through the two K buffers (tile j in buffer
    // j % 2, K_0 and K_1 already loaded) for the scores and their maximum;
    // then K_0 and K_1 are loaded again for the item itself.
    float m_exact = -INFINITY;
    if constexpr (FIXED) {
      if (exact) {
        for (int jj = 0; jj < n_tiles; ++jj) {
          if (jj > 0) wait_all();   // K_jj landed; every wave is done with tile jj-1
          if (jj > 0 && jj + 1 < n_tiles) load_k(krs, ((jj + 1) & 1) ? K1 : K0, jj + 1);
          w.scores(sa, (jj & 1) ? K1 : K0);
          apply_mask(sa, jj);
#pragma unroll
          for (int v = 0; v < W::NS; ++v) m_exact = __builtin_elementwise_maximum(m_exact, W::at(sa, v));
        }
        m_exact = pair_max(m_exact);
        wait_all();
        load_k(krs, K0, 0);
        if (1 < n_tiles) load_k(krs, K1, 1);
        wait_all();
      }
    }

    // ---- running state -------------------------------------------------------
    w.m = -INFINITY;
    w.l = 0.0f;
    w.lo = 0.0f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.oacc[t][r] = 0.0f;

    // Tiles no row of the workgroup needs masked run software-pipelined: step j
    // handles tile j and computes tile j+1's scores (and, in running-maximum
    // mode, maximum), so both must be such tiles; its loads (K_{j+2}, V_{j+1})
    // must not reach the tile that ends past N.  The rest run in a second loop.
    const int n_full = CAUSAL ? min(q0 / BC, N / BC) : N / BC;
    int n_pipe = max(0, min(n_full, n_tiles) - 1);
    if (n_tiles > N / BC) n_pipe = max(0, min(n_pipe, N / BC - 2));

    // On entry to step j the scores of tile j are in sa (masked) with the
    // reference maximum, mc and alpha set for it.  Step j (with the K stream
    // one tile ahead): wait for K_{j+1}, V_j; start K_{j+2}, V_{j+1}; compute.
    w.scores(sa, K0);
    apply_mask(sa, 0);
    if constexpr (FIXED) {
      // the reference is the first tile's maximum (or the exact one) for the
      // whole item; O, l, lo start at 0, so alpha never applies
      if (exact) {
        w.m = m_exact;
        w.mc = (m_exact == -INFINITY ? 0.0f : m_exact) * w.c;
      } else {
        // p_max * 2^-headroom for the first tile: later tiles may outgrow it
        // by 2^headroom before P nears the range bound
        w.max_all(sa);
        w.mc += p.headroom;
      }
      w.moved = false;
      w.alpha = 1.0f;
    } else {
      w.max_all(sa);
    }

    // Pipelined step j loads K_{j+2} (if any) into the K buffer tile j used and
    // V_{j+1} into the other V buffer, both wholly inside the sequence, one
    // 1 KiB piece at a time.  Even j: K_{j+1} is in K1, V_j in V0.
    // When step j has no K_{j+2} (the last step of an item whose tiles all
    // run here), its K loads still issue, through a copy of the K buffer
    // resource that spans no bytes: every access is out of range, no memory
    // is read, and the step needs no branch and no VALU per load.
    int j = 0;
    // the K loads of a step with no K_{j+2} go through a buffer of no bytes
    const u32x4 krs_void = (u32x4){krs[0], krs[1], 0u, krs[3]};
    u32x4 kstep = krs;
    auto ld_even = [&](int k) {
      if (k < PER_W) {
        load_one(kstep, K0 + wofs + k * 1024, koff_t(k), (j + 2) * TILE_BYTES + k * 1024);
      } else {
        load_one(vrs, V1 + wofs + (k - PER_W) * 1024, voff, (j + 1) * TILE_BYTES + (k - PER_W) * 1024);
      }
    };
    auto ld_odd = [&](int k) {
      if (k < PER_W) {
        load_one(kstep, K1 + wofs + k * 1024, koff_t(k), (j + 2) * TILE_BYTES + k * 1024);
      } else {
        load_one(vrs, V0 + wofs + (k - PER_W) * 1024, voff, (j + 1) * TILE_BYTES + (k - PER_W) * 1024);
      }
    };
    constexpr int NL = 2 * PER_W;
    // (the priority is set once per pair of steps: its branches would
    // otherwise split the pair's straight-line code in two)
    for (; j + 1 < n_pipe; j += 2) {
      progress(2);
      wait_all();
      kstep = j + 2 < n_tiles ? krs : krs_void;
      if constexpr (FIXED)   // no maximum, no rescale
        w.template pipe_tile_fixed<NL>(sa, sb, K1, V0, ld_even);
      else if (w.moved)
        w.template pipe_tile<true, NL>(sa, sb, K1, V0, ld_even);
      else
        w.template pipe_tile<false, NL>(sa, sb, K1, V0, ld_even);
      ++j;
      wait_all();
      kstep = j + 2 < n_tiles ? krs : krs_void;
      if constexpr (FIXED)
        w.template pipe_tile_fixed<NL>(sb, sa, K0, V1, ld_odd);
      else if (w.moved)
        w.template pipe_tile<true, NL>(sb, sa, K0, V1, ld_odd);
      else
        w.template pipe_tile<false, NL>(sb, sa, K0, V1, ld_odd);
      --j;
    }
    if (j < n_pipe) {
      wait_all();
      progress(1);
      kstep = j + 2 < n_tiles ? krs : krs_void;
      if constexpr (FIXED)
        w.template pipe_tile_fixed<NL>(sa, sb, K1, V0, ld_even);
      else if (w.moved)
        w.template pipe_tile<true, NL>(sa, sb, K1, V0, ld_even);
      else
        w.template pipe_tile<false, NL>(sa, sb, K1, V0, ld_even);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sa[kb] = sb[kb];
      ++j;
    }

    // ---- the remaining tiles: still pipelined with the next tile's scores,
    // but the next tile may need its mask (causal diagonal, keys past N)
    // before its maximum, and the loads may reach the tile that ends past N.
    // The buffers alternate at run time here.
    auto ld_any = [&](int k) {
      const bool odd = j & 1;
      if (k < PER_W) {
        // no K_{j+2}: the loads go through the empty resource, as in the pipelined steps
        load_one(j + 2 < n_tiles ? krs : krs_void, (odd ? K1 : K0) + wofs + k * 1024,
                 koff_t(k) + (j + 2 == j_tail ? tail_delta(k) : 0),
                 (j + 2) * TILE_BYTES + k * 1024);
      } else {
        const int t = k - PER_W;
        load_one(vrs, (odd ? V0 : V1) + wofs + t * 1024, voff + (j + 1 == j_tail ? tail_delta(t) : 0),
                 (j + 1) * TILE_BYTES + t * 1024);
      }
    };
    for (; j + 1 < n_tiles; ++j) {
      wait_all();
      progress(1);
      // causal: the next tile may be the last and wholly after this wave's
      // rows (then it is the item's last tile)
      const bool odd = j & 1;
      if constexpr (CAUSAL) {
        // a causal diagonal tile, masked in the pipeline (keys past N follow
        // every row below N, so the causal mask hides them as well)
        if constexpr (FIXED)
          w.template pipe_tile_fixed<NL, decltype(ld_any), true>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any,
                                                                 (j + 1) * BC - wr0);
        else if (w.moved)
          w.template pipe_tile<true, NL, decltype(ld_any), true, true>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any,
                                                                       (j + 1) * BC - wr0);
        else
          w.template pipe_tile<false, NL, decltype(ld_any), true, true>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any,
                                                                        (j + 1) * BC - wr0);
      } else {
        if constexpr (FIXED)
          w.template pipe_tile_fixed<NL>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any);
        else if (w.moved)
          w.template pipe_tile<true, NL, decltype(ld_any), false>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any);
        else
          w.template pipe_tile<false, NL, decltype(ld_any), false>(sa, sb, odd ? K0 : K1, odd ? V1 : V0, ld_any);
        apply_mask(sb, j + 1);
        if constexpr (!FIXED) w.max_all(sb);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sa[kb] = sb[kb];
    }


    // ---- the last tile: P V only -----------------------------------------------------
    wait_all();
    // Both K buffers, and the V buffer the last tile does not use, are free
    // now: start the next item's Q, K_0, K_1 and, when it is free, V_0.
    int bh2 = 0, qb2 = 0;
    const bool more = item(t_item + 1, bh2, qb2);
    const u32x4 krs2 = load_rsrc(p.k + (size_t)bh2 * N * D, HEAD_BYTES);
    const u32x4 vrs2 = load_rsrc(p.v + (size_t)bh2 * N * D, HEAD_BYTES);
    const int n_tiles2 = tiles_of(qb2);
    const bool last_odd = j & 1;
    if (more) {
      load_k(krs2, K0, 0);
      if (1 < n_tiles2) load_k(krs2, K1, 1);
      if (last_odd) load_v(vrs2, voff, V0, 0);
    }
    // ---- epilogue: O = acc / lo, LSE = ln2 * (mc + log2 l) --------------------
    // A lane holds 4-float pieces of one row of O, so storing from the
    // accumulators writes 32 bytes into each of 32 rows per instruction.
    // Instead each wave turns every 32x32 block of O row-major in a private
    // 4 KiB of LDS (16-byte chunk c of row r at chunk c ^ ((r/2) % 8), so
    // neither pattern has bank conflicts), and every store then writes 8
    // whole 128-byte row pieces.
    auto epilogue = [&](lds_u8* stage) {
      const float lt = pair_sum(w.l);
      const float inv = __builtin_amdgcn_rcpf(pair_sum(w.lo));
      // lane-derived offsets computed here, not hoisted out of the item loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int h = ln >> 5, r = ln & 31;         // accumulator side: row r, chunks 2i + h
      const int rs = ln >> 3, cs = ln & 7;        // store side: row 8s + rs, chunk cs
      typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
      // O of the head as a buffer: the rows past N-1 of a ragged last block
      // fall outside it and their stores are dropped
      const __amdgpu_buffer_rsrc_t ors = head_rsrc(p.o + head_off, (unsigned)N * D * 4);
      // unsigned byte offsets: the host admits heads whose fp32 O (plus the
      // rows of a ragged last block) spans up to 2^32 - 1 bytes
      const unsigned vo = (unsigned)(wr0 + rs) * (unsigned)(D * 4) + (unsigned)(cs * 16);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 val = {w.oacc[t][4 * i + 0] * inv, w.oacc[t][4 * i + 1] * inv,
                             w.oacc[t][4 * i + 2] * inv, w.oacc[t][4 * i + 3] * inv};
          *(lds_f32x4*)(stage + r * 128 + (((2 * i + h) ^ ((r >> 1) & 7)) << 4)) = val;
        }
#pragma unroll
        for (int s8 = 0; s8 < 4; ++s8) {
          const int row = 8 * s8 + rs;
          const f32x4 val = *(const lds_f32x4*)(stage + row * 128 + ((cs ^ ((row >> 1) & 7)) << 4));
          store_b128(ors, val, vo + (unsigned)(s8 * 8 * D * 4 + t * 128));
        }
      }
      if (qrow < N && lane < 32)
        p.lse[(size_t)bh * N + qrow] = (w.mc + __builtin_amdgcn_logf(lt)) * 0.69314718055994530942f;
    };
    // a wave whose rows all precede the tile's first key has nothing to do
    if (!CAUSAL || j * BC <= wr0 + 31) w.finish(sa, last_odd ? V1 : V0);
    if (more) load_q(bh2, qb2);   // the fragment registers are free from here on
    if (OWN_STAGE) {
      epilogue((lds_u8*)o_lds + wave * 4096);
    } else {
      // V buffer 1 takes the staging: when the last tile is even it held
      // tile j-1 and is free since the last tile's barrier; when it is odd
      // the other waves may still be reading it, so wait for them (a plain
      // barrier: __syncthreads() would also wait for the next item's loads,
      // none of which writes V buffer 1).
      if (last_odd) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
      }
      epilogue(V1 + wave * 4096);
    }
    if constexpr (FIXED) {
      // vote: some P (or a sum of P V) may have left its range
      if (!exact && __builtin_amdgcn_ballot_w64(!(w.lo <= p.l_max)) != 0 && lane == 0) redo_tag = t_item + 1;
    }
    if (!more) {
      if constexpr (!FIXED) break;
      if (exact) break;
      __syncthreads();   // every wave's tag is written
      if (__builtin_amdgcn_readfirstlane(redo_tag) != t_item + 1) break;
      ++t_item;          // the loop head computes item t_item - 1 again
      v0_late = false;
      continue;
    }
    ++t_item;
    bh = bh2;
    qb = qb2;
    krs = krs2;
    vrs = vrs2;
    n_tiles = n_tiles2;
    v0_late = !last_odd;
  }
}

// ---- launch ------------------------------------------------------------------

template <bool BF16, int D, bool CAUSAL, bool FIXED, int NW>
static const void* kernel_fn() {
  return reinterpret_cast<const void*>(&attn_fwd_kernel<BF16, D, CAUSAL, FIXED, NW>);
}

// Tile variants: 1 = 128-row items (4 waves), 2 = 256-row items (8 waves,
// fixed-reference mode only).
int block_rows(int tile) { return tile == 2 ? 256 : 128; }
static int tile_waves(int tile) { return tile == 2 ? 8 : 4; }

template <bool FIXED, int NW>
static const void* variant_fn_m(bool bf16, int d, bool causal) {
  return bf16 ? (d == 64 ? (causal ? kernel_fn<true, 64, true, FIXED, NW>() : kernel_fn<true, 64, false, FIXED, NW>())
                         : (causal ? kernel_fn<true, 128, true, FIXED, NW>() : kernel_fn<true, 128, false, FIXED, NW>()))
              : (d == 64 ? (causal ? kernel_fn<false, 64, true, FIXED, NW>() : kernel_fn<false, 64, false, FIXED, NW>())
                         : (causal ? kernel_fn<false, 128, true, FIXED, NW>() : kernel_fn<false, 128, false, FIXED, NW>()));
}

// The kernel of a (mode, tile) pair; the running-maximum mode exists for
// the 128-row tile only (the launcher's callers check that).
static const void* variant_fn(bool bf16, int d, bool causal, bool fixed, int tile) {
  if (!fixed) return variant_fn_m<false, 4>(bf16, d, causal);
  return tile == 2 ? variant_fn_m<true, 8>(bf16, d, causal) : variant_fn_m<true, 4>(bf16, d, causal);
}

// Workgroups of one kernel variant that the current device runs at once
// (compute units x workgroups per compute unit), cached per device.
static int resident_groups(int variant, const void* fn, int threads) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[32][kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cache[variant][dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess) return -1;
  const int n = std::max(1, cus) * std::max(1, per_cu);
  if (dev >= 0 && dev < kMaxDev) cache[variant][dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t kernel_info(bool bf16, int d, bool causal, bool fixed, int tile, KernelInfo& out) {
  const void* fn = variant_fn(bf16, d, causal, fixed, tile);
  hipFuncAttributes attr{};
  hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, tile_waves(tile) * 64, 0);
  if (e != hipSuccess) return e;
  out.rows = block_rows(tile);
  out.waves = tile_waves(tile);
  out.vgprs = attr.numRegs;
  out.lds_bytes = (int)attr.sharedSizeBytes;
  out.scratch_bytes = (int)attr.localSizeBytes;
  out.groups_per_cu = per_cu;
  return hipSuccess;
}

hipError_t resolve_cfg(bool bf16, int d, bool causal, const AttnParams& prm, LaunchCfg& cfg) {
  if (cfg.mode == 0) cfg.mode = 1;
  if (cfg.tile == 0) cfg.tile = 1;
  const bool fixed = cfg.mode == 1;
  if (!fixed && cfg.tile != 1) return hipErrorInvalidValue;
  const long long n_qblk = (prm.N + block_rows(cfg.tile) - 1) / block_rows(cfg.tile);
  const long long items = (long long)prm.BH * n_qblk;
  const int variant = (cfg.tile == 2 ? 16 : 0) + (fixed ? 8 : 0) + (bf16 ? 4 : 0) + (d == 128 ? 2 : 0) + (causal ? 1 : 0);
  const int slots = resident_groups(variant, variant_fn(bf16, d, causal, fixed, cfg.tile), tile_waves(cfg.tile) * 64);
  if (slots < 0) return hipErrorInvalidDevice;
  // built-in: heads split over the 8 XCDs when they divide evenly, as many
  // workgroups as run at once, groups of heads that fill one round of items.
  // With at least four items per resident workgroup, one domain and a grid
  // of twice the resident workgroups, groups of 8 heads, measured faster
  // (1-2 %: the second half of the grid is dispatched as the first half
  // finishes, which evens out the ends of the item lists); with fewer items
  // it is much slower.
  if (cfg.n_dom == 0 && cfg.n_work == 0 && items >= 4LL * slots) {
    cfg.n_dom = 1;
    cfg.n_work = 2 * slots;
    if (cfg.grp == 0) cfg.grp = 8;
  }
  if (cfg.n_dom == 0) cfg.n_dom = (prm.BH % 8 == 0) ? 8 : 1;
  if (cfg.n_dom == 8 && prm.BH % 8 != 0) cfg.n_dom = 1;
  const long long per_dom = items / cfg.n_dom;
  if (cfg.n_work == 0) cfg.n_work = std::max(1, slots / cfg.n_dom);
  cfg.n_work = (int)std::min<long long>(cfg.n_work, per_dom);
  if (cfg.grp == 0) cfg.grp = (int)std::max<long long>(1, cfg.n_work / n_qblk);
  cfg.grp = std::min(cfg.grp, prm.BH / cfg.n_dom);
  if (cfg.prio == 0) cfg.prio = 1;
  return hipSuccess;
}

hipError_t launch_attn_fwd(bool bf16, int d, bool causal, AttnParams prm, const LaunchCfg& cfg,
                           hipStream_t stream) {
  const int bm = block_rows(cfg.tile);
  prm.n_qblk = (prm.N + bm - 1) / bm;
  // raw-score margin before the reference maximum moves: 2^2 in probability
  // units for bf16, 2^8 for fp16 (O is divided by the sum of the rounded P,
  // so the margin changes no weight of O, only the range of P)
  prm.thr = fminf((bf16 ? 2.0f : 8.0f) / prm.c, 3.0e38f);
  // fixed-reference mode (cfg.mode 1) unless the caller asked for the
  // running maximum.  Bound on a lane's sum lo of the 16-bit P (so on each
  // of them) before the item is computed again: bf16 P keep fp32's exponent
  // range, and 2^48 leaves the P V sums far from overflow; fp16 P are finite
  // exactly when their sum is.
  const bool fixed = cfg.mode != 2;
  prm.l_max = bf16 ? 281474976710656.0f : 3.402823466e38f;
  // The fixed reference sits this many log2 units above the first tile's
  // maximum, so a row may outgrow its first tile by 2^(48 + 48) (bf16) or
  // 2^(16 + 4) (fp16) before its item is computed again.  The first tile's
  // largest p is then 2^-48: fp32 and bf16 keep 126 binades below 1, so the
  // terms that matter stay normal.  fp16 has 14, hence its smaller headroom.
  prm.headroom = bf16 ? 48.0f : 4.0f;
  const long long items = (long long)prm.BH * prm.n_qblk;
  if (items > (1LL << 30)) return hipErrorInvalidConfiguration;
  prm.n_dom = cfg.n_dom;
  prm.n_work = cfg.n_work;
  prm.grp = cfg.grp;
  prm.prio = cfg.prio == 1 ? 1 : 0;
  const int grid = prm.n_dom * prm.n_work;
  void* args[] = {&prm};
  return hipLaunchKernel(variant_fn(bf16, d, causal, fixed, cfg.tile), dim3(grid), dim3(tile_waves(cfg.tile) * 64),
                         args, 0, stream);
}

}  // namespace ttc
