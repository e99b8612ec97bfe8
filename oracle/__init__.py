"""fp64 CPU oracles for the attention forward pass and the row-wise softmax
(test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .attention import attention_online, attention_probs, attention_ref, attention_rows
from .softmax import softmax_rows_ref

__all__ = ["attention_ref", "attention_rows", "attention_online", "attention_probs", "softmax_rows_ref"]
