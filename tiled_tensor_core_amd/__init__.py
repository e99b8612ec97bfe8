"""MI355X-native fused FlashAttention forward (gfx950 HIP kernels behind a C ABI).

``attn_fwd`` and friends live in ``tiled_tensor_core_amd.attn`` and load the
compiled library on first use; importing this package loads nothing.
"""

__all__ = ["attn", "synth"]
