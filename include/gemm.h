/*
 * gemm.h -- C ABI of the MI355X (gfx950) tiled bf16 GEMM with a fused bias
 * + GELU epilogue.
 *
 * Operation (TileLang tutorial "Designing high-performance GPU kernels with
 * a high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
 * sections on the tiled tensor-core matrix multiplication and on the fused
 * GEMM epilogue): a linear layer
 *
 *     C[m, n] = epilogue( sum_k A[m, k] * W[n, k] + bias[n] )
 *
 * with the bias addition and the GELU activation applied to the fp32
 * accumulator in registers, before the single write of C.  GELU is the
 * exact form, GELU(z) = z * Phi(z) = z / 2 * erfc(-z / sqrt(2)), Phi the
 * standard normal distribution function.
 *
 * Arguments
 * ---------
 *   a         device pointer, read only: bf16 [M, K], row-major (K contiguous).
 *   w         device pointer, read only: bf16 [N, K], row-major (K contiguous),
 *             i.e. the weight of a linear layer with N outputs and K inputs.
 *   bias      device pointer, read only: fp32 [N]; may be NULL only with
 *             GEMM_EPI_NONE.
 *   c         device pointer, written: bf16 [M, N], row-major.  Every element
 *             is overwritten; values are rounded to nearest even.
 *   M, N, K   sizes: M >= 1; N >= 8 and a multiple of 8; K >= 8 and a
 *             multiple of 8; N and K at most 4194296 (256-row tiles are
 *             addressed with 32-bit byte offsets).
 *   epilogue  GEMM_EPI_NONE (C = A W^T), GEMM_EPI_BIAS (+ bias) or
 *             GEMM_EPI_BIAS_GELU (GELU(A W^T + bias)).
 *   stream    a hipStream_t passed as void* (NULL = the default stream).
 *
 * Arithmetic: products of bf16 values accumulated in fp32 by the matrix
 * cores, epilogue in fp32, one rounding to bf16 at the end.
 *
 * Ownership and execution: the caller allocates and owns every buffer; the
 * library allocates nothing and keeps no pointer after it returns.  The call
 * only enqueues work on `stream`.  c must not overlap a, w or bias.
 *
 * Alignment: every pointer must be 16-byte aligned.
 *
 * Errors: arguments are checked on the host before any HIP call and return
 * the attn_status codes of attn.h (ATTN_ERR_NULL, ATTN_ERR_SHAPE,
 * ATTN_ERR_ALIGN, ATTN_ERR_ALIAS, ATTN_ERR_CONFIG for an unknown epilogue;
 * ATTN_ERR_HIP when the launch fails, with the HIP error text in
 * attn_last_error()).
 */
#ifndef TTC_GEMM_H
#define TTC_GEMM_H

#ifdef __cplusplus
extern "C" {
#endif

enum gemm_epilogue { GEMM_EPI_NONE = 0, GEMM_EPI_BIAS = 1, GEMM_EPI_BIAS_GELU = 2 };

/* C = epilogue(A W^T + bias) in bf16 (see above).  Returns an attn_status code. */
int gemm_bf16(const void* a, const void* w, const float* bias, void* c, int M, int N, int K, int epilogue,
              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTC_GEMM_H */
