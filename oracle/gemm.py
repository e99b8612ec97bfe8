"""CPU oracle for the GEMM kernel with the fused bias + GELU epilogue.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests and the benchmark's CPU-baseline leg use
it.  It shares no code with the HIP kernels or their binding and works on
plain float64 arrays.

Source of the operation: the TileLang tutorial "Designing high-performance
GPU kernels with a high-level Python DSL via TVM: from tensor-core GEMM to
FlashAttention" (aioga.com, English text), the section on the tiled
tensor-core matrix multiplication and the following one on the fused GEMM
epilogue: the matrix product is extended by adding a bias and applying the
GELU activation to the accumulator while it is still in registers, before
the single write of the output, and the fused kernel is compared with eager
PyTorch.  The pages give no formula, layout, shape or type, so these
readings are taken:

* the product is a linear layer, ``C = A W^T`` with ``A`` of shape [M, K]
  and ``W`` of shape [N, K] (both contiguous along K), and the bias is a
  vector of N values added to every row: ``Z = A W^T + b``;
* GELU is the exact form eager PyTorch uses by default,
  ``GELU(z) = z * Phi(z) = z / 2 * (1 + erf(z / sqrt(2)))``, with Phi the
  standard normal distribution function (not the tanh approximation).  The
  oracle evaluates Phi(z) as ``erfc(-z / sqrt(2)) / 2``, the same function
  without the cancellation of ``1 + erf`` for large negative z;
* the epilogue is one of: none (``C = A W^T``), bias only, bias then GELU;
* the inputs are the already-rounded bf16 values of A and W and the fp32
  bias, upcast exactly; the oracle computes in float64.

Every function here is pinned by ``tests/test_gemm_oracle.py``.
"""

from __future__ import annotations

import numpy as np
from scipy.special import erfc

__all__ = ["EPI_NONE", "EPI_BIAS", "EPI_BIAS_GELU", "gelu_ref", "gemm_ref"]

EPI_NONE = 0
EPI_BIAS = 1
EPI_BIAS_GELU = 2


def gelu_ref(z) -> np.ndarray:
    """Exact GELU of an array, z * Phi(z), in float64."""
    z = np.asarray(z, dtype=np.float64)
    return z * (0.5 * erfc(-z / np.sqrt(2.0)))


def gemm_ref(a, w, bias=None, epilogue: int = EPI_BIAS_GELU) -> np.ndarray:
    """Epilogue(A W^T [+ b]) in float64 for A [M, K], W [N, K], b [N]."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if a.ndim != 2 or w.ndim != 2 or a.shape[1] != w.shape[1]:
        raise ValueError(f"expected A [M, K] and W [N, K], got {a.shape} and {w.shape}")
    if epilogue not in (EPI_NONE, EPI_BIAS, EPI_BIAS_GELU):
        raise ValueError(f"unknown epilogue {epilogue}")
    z = a @ w.T
    if epilogue == EPI_NONE:
        return z
    b = np.asarray(bias, dtype=np.float64)
    if b.shape != (w.shape[0],):
        raise ValueError(f"bias must have shape ({w.shape[0]},), got {b.shape}")
    z = z + b[None, :]
    if epilogue == EPI_BIAS:
        return z
    return gelu_ref(z)
