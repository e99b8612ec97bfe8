"""fp64 CPU oracles for the attention forward pass, the row-wise softmax and
the GEMM with its fused bias + GELU epilogue (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .attention import attention_online, attention_probs, attention_ref, attention_rows
from .gemm import EPI_BIAS, EPI_BIAS_GELU, EPI_NONE, gelu_ref, gemm_ref
from .softmax import softmax_rows_ref

__all__ = ["attention_ref", "attention_rows", "attention_online", "attention_probs", "softmax_rows_ref",
           "gemm_ref", "gelu_ref", "EPI_NONE", "EPI_BIAS", "EPI_BIAS_GELU"]
