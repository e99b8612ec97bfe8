// Un-fused attention forward for gfx950: the score matrix in device memory.
//
// Method: TileLang tutorial "Designing high-performance GPU kernels with a
// high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention".
// Its FlashAttention section builds the fused kernel so that the N x N score
// matrix never reaches global memory; this path is what that avoids, run as
// three kernels so its traffic and time can be measured beside the fused
// kernel's:
//   1. unf_scores: S = scale * Q K^T, fp32, causal entries above the
//      diagonal set to -inf, written to a workspace [B*H, N, N];
//   2. the row softmax of the tutorial's epilogue/softmax section
//      (softmax_kernel.hip), in place on S, which also writes each row's
//      natural log-sum-exp into lse;
//   3. unf_pv: O = P V, P rounded to the input type (as the fused kernel
//      rounds its probabilities) and fp32 accumulation on the matrix cores.
//
// Layout: q, k, v [B*H, N, D] 16-bit; S/P fp32 [B*H, N, N] (row stride N);
// o fp32 [B*H, N, D]; lse fp32 [B*H, N].
//
// Both kernels use v_mfma_f32_32x32x16_{bf16,f16}: a wave owns 32 query rows.
//   * scores: A = 32 rows of Q, B = 32 rows of K (8 consecutive head-dim
//     values per lane, straight from global memory), so lane l's
//     accumulator holds key l % 32 of rows 8(r/4) + 4(l/32) + r%4, and each
//     store instruction writes two whole 128-byte row pieces of S.  Tiles
//     wholly above a wave's rows (causal) are written as -inf without MFMAs.
//   * pv: A = 32 rows of P (8 keys per lane, converted to 16 bit with round
//     to nearest even), B = a 16-key slice of a V tile held in LDS and read
//     with the transposing ds_read_b64_tr_b16, the V tile swizzled so those
//     reads are free of bank conflicts; both operands take a lane's 8 keys in
//     the order that read delivers them.  Causal: key tiles past a
//     workgroup's last row hold P = 0 exactly and are skipped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "softmax_launch.h"
#include "unfused_launch.h"

namespace ttc_unf {

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
typedef __attribute__((address_space(3))) uint8_t lds_u8;

#define UNF_INLINE __device__ __attribute__((always_inline)) inline

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBM = kNW * 32;   // query rows per workgroup
constexpr int kBN = 64;         // keys per tile

template <bool BF16>
UNF_INLINE f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF16>
UNF_INLINE uint32_t pack2(float x, float y) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
}

// 16-byte chunk ch of V-tile row r is stored at chunk ch ^ vswz(r): the
// transposing reads below then touch every bank once per phase.
template <int D>
UNF_INLINE int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// ---- 1. scores ----------------------------------------------------------------
// Grid (ceil(N/64) key tiles, ceil(N/128) query blocks, B*H); 4 waves.
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(kNW * 64) unf_scores(UnfParams p) {
  constexpr int DK = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N;
  const int c0 = blockIdx.x * kBN;
  const int wr0 = blockIdx.y * kBM + wave * 32;
  if (wr0 >= N) return;   // every row of this wave is past the sequence (no barrier follows)
  const size_t bh = blockIdx.z;
  float* S = p.s + bh * (size_t)N * (size_t)N;
  const int col = lane & 31;      // key column of the accumulator (within a 32-key block)
  const int half = lane >> 5;     // rows 4*half + ... of the accumulator

  // row i, key j of block kb for accumulator register r
  auto row_of = [&](int r) { return wr0 + 8 * (r >> 2) + 4 * half + (r & 3); };

  if (CAUSAL && c0 > wr0 + 31) {   // every key of the tile follows every row of the wave
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int j = c0 + 32 * kb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = row_of(r);
        if (i < N && j < N) __builtin_nontemporal_store(-INFINITY, S + (size_t)i * N + j);
      }
    }
    return;
  }
  const uint16_t* qh = p.q + bh * (size_t)N * D;
  const uint16_t* kh = p.k + bh * (size_t)N * D;
  // A: query row wr0 + lane%32 (rows past N repeat row N-1; not stored)
  const int qr = min(wr0 + col, N - 1);
  u32x4 qa[DK];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) qa[kk] = *reinterpret_cast<const u32x4*>(qh + (size_t)qr * D + 16 * kk + 8 * half);
  f32x16 acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // B: key row c0 + 32 kb + lane%32 (rows past N repeat row N-1; not stored)
    const int kr = min(c0 + 32 * kb + col, N - 1);
    acc[kb] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      acc[kb] = mfma<BF16>(qa[kk], *reinterpret_cast<const u32x4*>(kh + (size_t)kr * D + 16 * kk + 8 * half), acc[kb]);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = c0 + 32 * kb + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row_of(r);
      const float sv = (CAUSAL && j > i) ? -INFINITY : acc[kb][r] * p.scale;
      if (i < N && j < N) __builtin_nontemporal_store(sv, S + (size_t)i * N + j);
    }
  }
}

// ---- 3. O = P V -------------------------------------------------------------------
// Grid (ceil(N/128) query blocks, B*H); 4 waves.  A workgroup streams the
// key tiles its rows can see; V tile j goes through LDS, P straight from
// device memory into the A operand.
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(kNW * 64) unf_pv(UnfParams p) {
  constexpr int DT = D / 32;
  constexpr int ROW_BYTES = 2 * D;
  constexpr int CPR = D / 8;   // 16-byte chunks per V row
  __shared__ __attribute__((aligned(1024))) uint8_t vt_lds[kBN * ROW_BYTES];
  lds_u8* const vt = (lds_u8*)vt_lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N;
  const int q0 = blockIdx.x * kBM;
  const size_t bh = blockIdx.y;
  const int wr0 = q0 + wave * 32;
  const float* P = p.s + bh * (size_t)N * (size_t)N;
  const uint16_t* vh = p.v + bh * (size_t)N * D;
  const int n_keys = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (n_keys + kBN - 1) / kBN;
  const int col = lane & 31, half = lane >> 5;
  // A operand: P row wr0 + lane%32 (rows past N repeat row N-1; not stored)
  const int pr = min(wr0 + col, N - 1);
  const float* prow = P + (size_t)pr * N;
  const bool vec = (N & 3) == 0;   // P rows start 16-byte aligned
  // B operand (V[16 keys][32 dims] slice, transposed by the LDS read): lane
  // offsets within a V tile, per 32-dim block t
  int vro[DT];
  {
    const int g = lane >> 4, gj = lane & 15;
    const int vkey = 4 * (g >> 1) + (gj >> 2);          // + 16 * step (and + 8)
    const int vcol = 16 * (g & 1) + 4 * (gj & 3);       // + 32 t
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int c = 32 * t + vcol;
      vro[t] = vkey * ROW_BYTES + (((c >> 3) ^ vswz<D>(vkey)) << 4) + ((c & 7) << 1);
    }
  }
  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = (f32x16){};

  for (int jt = 0; jt < n_tiles; ++jt) {
    const int c0 = jt * kBN;
    __syncthreads();   // every wave is done reading the previous tile
#pragma unroll
    for (int idx = threadIdx.x; idx < kBN * CPR; idx += kNW * 64) {
      const int r = idx / CPR, ch = idx % CPR;
      const int gr = min(c0 + r, N - 1);   // rows past N: finite values, P = 0 for them
      const u32x4 val = *reinterpret_cast<const u32x4*>(vh + (size_t)gr * D + ch * 8);
      *(__attribute__((address_space(3))) u32x4*)(vt + r * ROW_BYTES + ((ch ^ vswz<D>(r)) << 4)) = val;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      // the transposing V read gives lane l, element e, the key
      // 8 (e / 4) + 4 (l / 32) + e % 4 of the 16-key step; P takes the same
      // keys, so the MFMA's sum over k pairs them up
      const int kb0 = c0 + 16 * ks + 4 * half, kb1 = kb0 + 8;
      float pv[8];
      if (vec && kb1 + 4 <= N) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(prow + kb0);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(prow + kb1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = a0[e];
          pv[4 + e] = a1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = (kb0 + e < N) ? prow[kb0 + e] : 0.0f;
          pv[4 + e] = (kb1 + e < N) ? prow[kb1 + e] : 0.0f;
        }
      }
      const u32x4 a = {pack2<BF16>(pv[0], pv[1]), pack2<BF16>(pv[2], pv[3]), pack2<BF16>(pv[4], pv[5]),
                       pack2<BF16>(pv[6], pv[7])};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const lds_u8* pa = vt + vro[t] + 16 * ks * ROW_BYTES;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * ROW_BYTES));
        const u32x4 b = {__builtin_bit_cast(uint32_t, (i16x2){lo[0], lo[1]}),
                         __builtin_bit_cast(uint32_t, (i16x2){lo[2], lo[3]}),
                         __builtin_bit_cast(uint32_t, (i16x2){hi[0], hi[1]}),
                         __builtin_bit_cast(uint32_t, (i16x2){hi[2], hi[3]})};
        acc[t] = mfma<BF16>(a, b, acc[t]);
      }
    }
  }
  // O row i, dim 32 t + lane%32 for accumulator register r: each store
  // instruction writes two whole 128-byte row pieces
  float* O = p.o + bh * (size_t)N * D;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = wr0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (i < N) __builtin_nontemporal_store(acc[t][r], O + (size_t)i * D + 32 * t + col);
    }
}

// ---- launch ------------------------------------------------------------------------

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_t(const UnfParams& prm, int BH, float* lse, hipStream_t stream) {
  const int N = prm.N;
  const dim3 block(kNW * 64);
  hipLaunchKernelGGL((unf_scores<BF16, D, CAUSAL>), dim3((N + kBN - 1) / kBN, (N + kBM - 1) / kBM, BH), block, 0,
                     stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = ttc_sm::launch_softmax(0, prm.s, prm.s, BH * N, N, lse, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((unf_pv<BF16, D, CAUSAL>), dim3((N + kBM - 1) / kBM, BH), block, 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_unfused(bool bf16, int d, bool causal, const UnfParams& prm, int BH, float* lse,
                          hipStream_t stream) {
  if (bf16) {
    if (d == 64) return causal ? launch_t<true, 64, true>(prm, BH, lse, stream) : launch_t<true, 64, false>(prm, BH, lse, stream);
    return causal ? launch_t<true, 128, true>(prm, BH, lse, stream) : launch_t<true, 128, false>(prm, BH, lse, stream);
  }
  if (d == 64) return causal ? launch_t<false, 64, true>(prm, BH, lse, stream) : launch_t<false, 64, false>(prm, BH, lse, stream);
  return causal ? launch_t<false, 128, true>(prm, BH, lse, stream) : launch_t<false, 128, false>(prm, BH, lse, stream);
}

// ---- the scratch of the allocation-free entry point ----------------------------
// A fixed-size score buffer in the library's own device memory, for callers
// that cannot allocate.  Every device the library runs on holds one copy
// until the process ends.  In host code `scratch` only stands for the symbol:
// its device address, different on each device, comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / 4];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace ttc_unf
