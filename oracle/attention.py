"""CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP kernels or their
binding and takes plain float64 arrays, so it never sees a device buffer.

Source of the method: the TileLang tutorial "Designing high-performance GPU
kernels with a high-level Python DSL via TVM: from tensor-core GEMM to
FlashAttention" (aioga.com, English text), section on the fused
FlashAttention forward kernel.  That section fixes

* the result: attention as computed by PyTorch's scaled dot-product attention,
  causal and non-causal, i.e. ``softmax(scale * Q K^T [+ causal mask]) V``;
* the method: Q/K/V are processed tile by tile, the full score matrix is never
  materialised, and an online softmax is maintained with a running maximum,
  a running normalisation sum and a rescaling factor, with the two products
  done as tiled matrix multiplications.

The pages print no formulas, so every step below is the plain definition of
the operation.  The readings taken where the pages are silent:

* ``scale`` is a caller argument (the pages never state it); it multiplies
  the fp64 scores, inputs are never pre-scaled.
* causal means key ``j`` is visible to query ``i`` iff ``j <= i`` (with equal
  query and key lengths top-left and bottom-right alignment coincide).
* a masked score is exactly ``-inf`` (its weight is exactly 0).
* the log-sum-exp output is in natural log: ``LSE_i = m_i + ln(l_i)``.
* the inputs are the already-rounded bf16/fp16 values, upcast exactly.

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, invariants, a 50-digit evaluation and PyTorch's CPU SDPA.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention_ref",
    "attention_rows",
    "attention_online",
    "attention_probs",
]


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float64:
        # every bf16/fp16/fp32 value is exactly representable in float64
        x = x.astype(np.float64)
    return x


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must all be [B, H, N, d]; got {q.shape}, {k.shape}, {v.shape}")


def _head_rows(qh, kh, vh, rows, causal, scale):
    """Exact attention for the query rows ``rows`` of one (b, h) head.

    qh, kh, vh: float64 [N, d]; rows: int array of query indices.
    Returns (O [len(rows), d], LSE [len(rows)]).

    Follows the definition the FlashAttention section validates against
    (scaled dot-product attention): S = scale * Q K^T, causal entries j > i
    set to -inf, P = exp(S - rowmax) / rowsum, O = P V, LSE = rowmax + ln(rowsum).
    """
    n = kh.shape[0]
    s = scale * (qh[rows] @ kh.T)                      # [r, N] scores
    if causal:
        key_idx = np.arange(n)[None, :]
        s = np.where(key_idx > rows[:, None], -np.inf, s)
    m = s.max(axis=1)                                  # row maximum
    e = np.exp(s - m[:, None])                         # exp(-inf) == 0 exactly
    l = e.sum(axis=1)                                  # normalisation sum
    p = e / l[:, None]                                 # probabilities
    o = p @ vh
    lse = m + np.log(l)
    return o, lse


def attention_ref(q, k, v, causal: bool, scale: float, row_chunk: int = 512):
    """One-shot fp64 attention forward over all heads.

    q, k, v: [B, H, N, d] arrays (any float dtype; upcast exactly to float64).
    Returns (O float64 [B, H, N, d], LSE float64 [B, H, N]).
    Query rows are processed ``row_chunk`` at a time only to bound memory;
    each chunk is the full definition (no online recurrence).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check_shapes(q, k, v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                o[b, h, rows], lse[b, h, rows] = _head_rows(
                    q[b, h], k[b, h], v[b, h], rows, causal, scale)
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows):
    """Exact fp64 output for chosen query rows of head (b, h) only.

    Used to check sampled outputs at sizes where the whole tensor would take
    the oracle too long.  Same definition as ``attention_ref``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = _as_f64(q[b, h])
    kh = _as_f64(k[b, h])
    vh = _as_f64(v[b, h])
    return _head_rows(qh, kh, vh, rows, causal, scale)


def attention_probs(q, k, causal: bool, scale: float):
    """The full probability matrix P [B, H, N, N] (small N only)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, N, d = q.shape
    p = np.empty((B, H, N, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(np.triu(np.ones((N, N), dtype=bool), 1), -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p[b, h] = e / e.sum(axis=1, keepdims=True)
    return p


def attention_online(q, k, v, causal: bool, scale: float, tile: int):
    """The tile-by-tile online-softmax recurrence, in fp64.

    This is the method the FlashAttention section describes: keys and values
    are visited one tile of ``tile`` keys at a time (the last tile may be
    ragged) and, for every query row, a running maximum ``m``, a running
    normalisation sum ``l`` and an unnormalised output ``acc`` are updated:

        m_new = max(m, max_j s_j)
        alpha = exp(m - m_new)            (0 while m is still -inf)
        p_j   = exp(s_j - m_new)
        l     = alpha * l + sum_j p_j
        acc   = alpha * acc + sum_j p_j v_j
        m     = m_new

    and at the end O = acc / l, LSE = m + ln(l).  Rows are vectorised with
    numpy; tiles are a Python loop, so use it on small shapes only.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check_shapes(q, k, v)
    if tile < 1:
        raise ValueError("tile must be >= 1")
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for c0 in range(0, N, tile):
                cols = np.arange(c0, min(N, c0 + tile))
                s = scale * (q[b, h] @ k[b, h, cols].T)          # [N, |tile|]
                if causal:
                    s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                m_new = np.maximum(m, s.max(axis=1))
                # a row whose every key so far is masked keeps m = -inf;
                # its factor and probabilities are 0, never NaN.
                live = np.isfinite(m_new)
                alpha = np.where(np.isfinite(m), np.exp(np.where(live, m - m_new, 0.0)), 0.0)
                p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, cols]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse

