"""fp64 CPU oracle for the attention forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .attention import attention_online, attention_probs, attention_ref, attention_rows

__all__ = ["attention_ref", "attention_rows", "attention_online", "attention_probs"]
