/*
 * softmax.h -- C ABI of the MI355X (gfx950) row-wise softmax kernel.
 *
 * Operation (TileLang tutorial "Designing high-performance GPU kernels with
 * a high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
 * section on the fused GEMM epilogue and the row-wise softmax): for every
 * row i of a [rows, cols] matrix x,
 *
 *     y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i),   m_i = max_k x_ik
 *
 * with the row maximum and the row sum found by reductions over register
 * fragments, so each row is read from device memory once (rows of up to
 * 16 KiB) and written once.
 *
 * Arguments
 * ---------
 *   x        device pointer, read only: contiguous [rows, cols] array, row
 *            stride cols elements, of type `dtype`.
 *   y        device pointer, written: same shape, layout and type as x.
 *            y may be x itself (in place); any other overlap is an error.
 *   rows     number of rows, >= 1.
 *   cols     number of columns, >= 1; one row must stay below 2 GiB.
 *   dtype    SOFTMAX_F32, SOFTMAX_BF16 or SOFTMAX_FP16.  Arithmetic is fp32
 *            throughout; 16-bit outputs are rounded to nearest even.
 *   stream   a hipStream_t passed as void* (NULL = the default stream).
 *
 * Values: an entry of -inf gets weight exactly 0.  A row whose entries are
 * all -inf has no softmax and comes out NaN, as does a row holding a NaN.
 * A row holding +inf comes out NaN (inf - inf).
 *
 * Ownership and execution: the caller allocates and owns both buffers; the
 * library allocates nothing and keeps no pointer after it returns.  The call
 * only enqueues work on `stream`.
 *
 * Alignment: x and y must be 16-byte aligned.  Rows of any length are read
 * with 16-byte loads where they are 16-byte aligned (rows whose byte length
 * is not a multiple of 16 start at every alignment: their head and tail,
 * under 16 bytes each, are read element by element); rows of odd byte
 * length longer than 16 KiB take a slower element-wise path.
 *
 * Errors: arguments are checked on the host before any HIP call and return
 * the attn_status codes of attn.h (ATTN_ERR_NULL, ATTN_ERR_SHAPE,
 * ATTN_ERR_ALIGN, ATTN_ERR_DTYPE, ATTN_ERR_ALIAS; ATTN_ERR_HIP when the
 * launch fails, with the HIP error text in attn_last_error()).
 */
#ifndef TTC_SOFTMAX_H
#define TTC_SOFTMAX_H

#ifdef __cplusplus
extern "C" {
#endif

enum softmax_dtype { SOFTMAX_F32 = 0, SOFTMAX_BF16 = 1, SOFTMAX_FP16 = 2 };

/* Row-wise softmax of x into y (see above).  Returns an attn_status code. */
int softmax_rows(const void* x, void* y, int rows, int cols, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTC_SOFTMAX_H */
