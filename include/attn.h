/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward pass.
 *
 * Operation (TileLang tutorial "Designing high-performance GPU kernels with
 * a high-level Python DSL via TVM: from tensor-core GEMM to FlashAttention",
 * section on the fused FlashAttention forward kernel): for every batch b and
 * head h,
 *
 *     O   = softmax(scale * Q K^T  [+ causal mask]) V
 *     LSE = log(sum_j exp(scale * q_i . k_j))      (natural log, visible j only)
 *
 * computed tile by tile with an online softmax (running row maximum, running
 * normalisation sum, rescaling factor), so the N x N score matrix never
 * reaches device memory.  The same section validates the kernel against
 * PyTorch's scaled dot-product attention, causal and non-causal; these
 * entry points follow its semantics (equal head counts, no dropout, no bias).
 *
 * Arguments common to every entry point
 * -------------------------------------
 *   q, k, v  device pointers, read only.  Each is a contiguous [B, H, N, d]
 *            array of 16-bit floats (bf16 or fp16, see the entry point), d
 *            fastest: element (b, h, n, c) is at ((b*H + h)*N + n)*d + c.
 *   o        device pointer, written: fp32 [B, H, N, d], same layout.
 *   lse      device pointer, written: fp32 [B, H, N], natural-log
 *            log-sum-exp of the scaled, masked scores of each query row.
 *   B, H, N  batch, heads, sequence length (queries = keys = N), each >= 1.
 *   d        head dimension: 64 or 128.
 *   causal   0: every key is visible; 1: key j is visible to query i iff
 *            j <= i.
 *   scale    finite multiplier of the scores (1/sqrt(d) for the usual
 *            attention); any sign, zero included.
 *   stream   a hipStream_t passed as void* (NULL = the default stream).
 *
 * Ownership and execution: the caller allocates and owns every buffer; the
 * library allocates nothing and keeps no pointer after it returns.  The call
 * only enqueues work on `stream` and returns; buffers must stay alive until
 * that stream has finished it.  Every row n < N of o and lse is overwritten.
 * o and lse must not overlap each other or the inputs.
 *
 * Alignment: every pointer must be 16-byte aligned.
 *
 * Errors: arguments are checked on the host before any HIP call; a failed
 * check returns its code and touches nothing.  ATTN_ERR_HIP means the launch
 * itself failed; attn_last_error() then returns the HIP error text for the
 * calling thread.  The functions are stateless and may be called from
 * several threads at once.
 */
#ifndef TTC_ATTN_H
#define TTC_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,           /* a pointer argument is NULL                     */
  ATTN_ERR_SHAPE = 2,          /* B, H or N < 1, B*H*N*d too large, or one head's
                                  fp32 O with 128 rows of margin,
                                  (N + 128) * d * 4 bytes, above 2^32 - 1      */
  ATTN_ERR_UNSUPPORTED_D = 3,  /* d is not 64 or 128                             */
  ATTN_ERR_ALIGN = 4,          /* a pointer is not 16-byte aligned               */
  ATTN_ERR_DTYPE = 5,          /* dtype code is not ATTN_BF16 or ATTN_FP16       */
  ATTN_ERR_HIP = 6,            /* the kernel launch failed (see attn_last_error) */
  ATTN_ERR_SCALE = 7,          /* scale is NaN or infinite                       */
  ATTN_ERR_CAUSAL = 8,         /* causal is not 0 or 1                           */
  ATTN_ERR_ALIAS = 9,          /* o or lse overlaps another buffer               */
  ATTN_ERR_CONFIG = 10,        /* a launch configuration field is out of range   */
  ATTN_ERR_WORKSPACE = 11,     /* workspace NULL, too small or misaligned        */
  ATTN_ERR_SCRATCH = 12        /* shape needs more than the built-in scratch     */
};

enum attn_dtype { ATTN_BF16 = 0, ATTN_FP16 = 1 };

/* Attention forward on bf16 q, k, v (FlashAttention section of the TileLang
 * tutorial).  Returns an attn_status code. */
int attn_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse,
                  int B, int H, int N, int d, int causal, float scale, void* stream);

/* The same on fp16 q, k, v. */
int attn_fwd_fp16(const void* q, const void* k, const void* v, float* o, float* lse,
                  int B, int H, int N, int d, int causal, float scale, void* stream);

/* The same, with the element type of q, k, v given by `dtype`
 * (ATTN_BF16 or ATTN_FP16). */
int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int H, int N, int d, int causal, float scale, void* stream, int dtype);

/* Launch configuration of the attention kernel.
 *
 * The tutorial's sections on schedule exploration and on autotuning build
 * several configurations of a kernel, benchmark each, check its output and
 * keep the fastest per workload.  The tile of this kernel (128 query rows x
 * 64 keys x d) is fixed by its hand-written instruction schedule, so the
 * configuration here is the launch schedule around that tile:
 *
 *   n_dom   head domains: 8 splits the B*H heads into 8 equal sets, one per
 *           XCD, so a head's K and V stay in one L2 (needs B*H % 8 == 0);
 *           1 lets every workgroup take items of any head.
 *   n_work  persistent workgroups per domain, 1 .. ATTN_MAX_WORKGROUPS;
 *           more than the domain's items (B*H/n_dom * ceil(N/128)) are
 *           clamped to that count.
 *   grp     heads per group in a domain's item order (items are listed
 *           group by group, longest first within a group); clamped to the
 *           heads of a domain.
 *   prio    ATTN_PRIO_ON: each workgroup raises its wave priority while it
 *           is behind on its item list, so the two workgroups sharing a
 *           compute unit finish together; ATTN_PRIO_OFF: constant priority.
 *
 *   mode    the exponent reference of the online softmax (attn_ref_mode
 *           below).
 *   tile    the tile variant (attn_tile below).
 *
 * A field of 0 (ATTN_PRIO_DEFAULT for prio) takes the built-in choice.  The
 * fields other than mode and tile change only which workgroup computes which
 * (head, query block) item and in what order, never an item's arithmetic:
 * every valid configuration of one (mode, tile) gives bit-identical o and
 * lse.  Different modes and tiles differ in rounding only. */
#define ATTN_MAX_WORKGROUPS (1 << 20)
enum attn_prio { ATTN_PRIO_DEFAULT = 0, ATTN_PRIO_ON = 1, ATTN_PRIO_OFF = 2 };

/* Exponent reference of the online softmax (the `mode` field).  Both modes
 * divide O by the sum of the 16-bit probabilities that multiply V, so O is
 * a weighted mean of the rows of V whatever the reference, and LSE uses the
 * sum of the unrounded fp32 probabilities.  The modes differ only in
 * rounding, within the same accuracy.
 *   ATTN_REF_FIXED    each (head, 128-row block) takes the maximum score of
 *                     each row over its first 64-key tile, raised by 48
 *                     (bf16) or 4 (fp16) in log2 units, as that row's
 *                     reference for all its tiles: no per-tile maximum, no
 *                     rescale of O.  A block in which a sum of 16-bit
 *                     probabilities passes 2^48 (bf16) or overflows (fp16),
 *                     or turns NaN, is computed again within the same launch
 *                     with each row's exact maximum (found by a pass over the
 *                     block's keys) as its reference.  The built-in choice.
 *   ATTN_REF_RUNNING  the reference follows the running maximum of every
 *                     32-row wave, moved (and O rescaled) only when a row
 *                     outgrows it by 2^2 (bf16) or 2^8 (fp16). */
enum attn_ref_mode { ATTN_REF_DEFAULT = 0, ATTN_REF_FIXED = 1, ATTN_REF_RUNNING = 2 };

/* Tile variant (the `tile` field): query rows per work item and waves per
 * workgroup.
 *   ATTN_TILE_128  128 rows, 4 waves of 32 rows, two workgroups per compute
 *                  unit.  The built-in choice.
 *   ATTN_TILE_256  256 rows, 8 waves, one workgroup per compute unit: each
 *                  K/V tile brought into LDS serves twice the rows, at the
 *                  price of wider causal diagonals and 8-wave barriers.
 *                  ATTN_REF_FIXED mode only. */
enum attn_tile { ATTN_TILE_DEFAULT = 0, ATTN_TILE_128 = 1, ATTN_TILE_256 = 2 };

typedef struct attn_launch_cfg {
  int n_dom;
  int n_work;
  int grp;
  int prio;
  int mode;   /* attn_ref_mode */
  int tile;   /* attn_tile */
} attn_launch_cfg;

/* Compiled resources of one kernel variant, as the device reports them. */
typedef struct attn_tile_resources {
  int rows;            /* query rows per work item                          */
  int waves;           /* waves per workgroup                               */
  int vgprs;           /* vector registers per lane                         */
  int lds_bytes;       /* static LDS per workgroup                          */
  int scratch_bytes;   /* scratch (spilled registers) per lane; 0 by design */
  int groups_per_cu;   /* workgroups a compute unit runs at once            */
} attn_tile_resources;

/* Resources of the kernel attn_fwd_cfg runs for (tile, mode, dtype, d,
 * causal) on the current device (fields of 0 mean the built-in choice), so
 * a search can drop variants that spill or exceed the LDS.  Queries the
 * device; enqueues nothing.  Errors: ATTN_ERR_NULL, _DTYPE, _UNSUPPORTED_D,
 * _CAUSAL, _CONFIG (no such variant), _HIP (query failed). */
int attn_tile_info(int tile, int mode, int dtype, int d, int causal, attn_tile_resources* out);

/* attn_fwd with an explicit launch configuration; cfg NULL is attn_fwd.
 * The caller owns cfg; it is read during the call only.  A field out of
 * range returns ATTN_ERR_CONFIG before any HIP call. */
int attn_fwd_cfg(const void* q, const void* k, const void* v, float* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, void* stream, int dtype,
                 const attn_launch_cfg* cfg);

/* Resolve a configuration for a shape on the current device, in place:
 * fields of 0 become the built-in choice, the others are clamped as
 * attn_fwd_cfg would clamp them.  Queries the device's occupancy (one HIP
 * call, cached per device); enqueues nothing.  Returns an attn_status code
 * (ATTN_ERR_HIP if the device query fails). */
int attn_resolve_cfg(int B, int H, int N, int d, int causal, int dtype, attn_launch_cfg* cfg);

/* Un-fused attention forward: the same operation, outputs and argument
 * rules as attn_fwd, computed the way the FlashAttention section of the
 * TileLang tutorial says the fused kernel avoids -- with the N x N score
 * matrix in device memory.  Three kernels run on `stream`:
 *   1. S = scale * Q K^T in fp32 (causal: -inf above the diagonal) into the
 *      workspace, as a [B*H, N, N] row-major array;
 *   2. the row softmax of softmax.h, in place on S, which also writes lse;
 *   3. O = P V, P rounded to q's type (as the fused kernel rounds its
 *      probabilities), fp32 accumulation.
 * It exists to measure what fusion saves (its S traffic is 16 B*H*N^2
 * bytes), and as a second, independent HIP path for the same result.
 *
 *   workspace        device pointer, 16-byte aligned, at least
 *                    attn_unfused_workspace_bytes(B, H, N) bytes; owned by
 *                    the caller, overwritten, must not overlap q, k, v, o,
 *                    lse; the stream must finish with it before it is reused.
 *   workspace_bytes  its size in bytes.
 * Limits beyond attn_fwd's: B*H <= 65535 and B*H*N < 2^31.  Errors: as
 * attn_fwd, plus ATTN_ERR_WORKSPACE (NULL, misaligned or too small; no
 * device work is enqueued). */
int attn_fwd_unfused(const void* q, const void* k, const void* v, float* o, float* lse,
                     void* workspace, unsigned long long workspace_bytes, int B, int H, int N,
                     int d, int causal, float scale, void* stream, int dtype);

/* Bytes of workspace attn_fwd_unfused needs: B*H*N*N*4 (0 if the shape is
 * outside its limits). */
unsigned long long attn_unfused_workspace_bytes(int B, int H, int N);

/* attn_fwd_unfused without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the score matrix goes to a fixed scratch
 * buffer of ATTN_UNFUSED_SCRATCH_BYTES (64 MiB) inside the library, one per
 * device, held from the first call until the process ends.  The call
 * allocates nothing; it looks the buffer's address up once per device (on
 * its first call there).  Shapes whose B*H*N*N*4 exceeds the buffer return
 * ATTN_ERR_SCRATCH before any HIP call.  Every call on a device uses that
 * device's one buffer and leaves its contents behind: calls that overlap on
 * one device (other streams, other threads) race and give wrong results.
 * Otherwise the same arguments, limits and errors as attn_fwd_unfused. */
#define ATTN_UNFUSED_SCRATCH_BYTES (64ull << 20)
int attn_fwd_unfused_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                             int B, int H, int N, int d, int causal, float scale, void* stream,
                             int dtype);

/* Static text for a status code ("unknown status" for other values). */
const char* attn_status_str(int status);

/* Text of the last HIP error a call on this thread returned ATTN_ERR_HIP
 * for ("" if none).  Valid until the next call on this thread. */
const char* attn_last_error(void);

/* Query rows of one work item of the kernel for head dim d (0 if d is
 * unsupported): there are B*H*ceil(N / rows) items, which the kernel's
 * workgroups (as many as the device runs at once) share out. */
int attn_block_rows(int d);

#ifdef __cplusplus
}
#endif

#endif /* TTC_ATTN_H */
