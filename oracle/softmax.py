"""CPU oracle for the row-wise softmax kernel.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests and the benchmark's CPU-baseline leg use
it.  It shares no code with the HIP kernels or their binding and works on
plain float64 arrays.

Source of the operation: the TileLang tutorial "Designing high-performance
GPU kernels with a high-level Python DSL via TVM: from tensor-core GEMM to
FlashAttention" (aioga.com, English text), section on the fused GEMM
epilogue and the row-wise softmax: a softmax along each row of a matrix,
with the row maximum and the row sum found by reductions over register
fragments.  The pages give no formula, no shapes and no types, so the
operation is the plain definition, and these readings are taken:

* the softmax runs along the last (contiguous) axis of a 2-D [rows, cols]
  matrix: ``y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i)`` with
  ``m_i = max_k x_ik`` (subtracting the row maximum changes nothing
  mathematically and keeps every exponent <= 0);
* an entry of ``-inf`` gets weight exactly 0; a row whose entries are all
  ``-inf`` has no defined softmax and yields NaN (0/0), as PyTorch does;
* the input is the already-rounded bf16/fp16/fp32 value, upcast exactly.

Every function here is pinned by ``tests/test_softmax_oracle.py``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["softmax_rows_ref"]


def softmax_rows_ref(x) -> np.ndarray:
    """Row softmax of a 2-D array in float64 (returns a new [rows, cols] array)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError(f"expected a 2-D [rows, cols] array, got shape {x.shape}")
    if x.shape[1] == 0:
        return np.zeros_like(x)
    with np.errstate(invalid="ignore"):
        m = x.max(axis=1)
        e = np.exp(x - m[:, None])
        s = e.sum(axis=1)
        y = e / s[:, None]
    return y
