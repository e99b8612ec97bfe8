"""Seeded synthetic Q/K/V inputs, shared by the tests, the benchmark and the
smoke check.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to the storage type and converts storage bits to other types.

Recipe (the same on every machine and numpy version):

* each tensor gets its own counter-based Philox-4x64 stream, keyed by
  ``(seed, tensor id)`` with tensor ids Q=0, K=1, V=2;
* the raw 64-bit words are turned into uniforms ``u = ((w >> 11) + 0.5) * 2^-53``
  in (0, 1), so no library distribution code is involved;
* normal draws use the Box-Muller transform on consecutive word pairs
  (``r = sqrt(-2 ln u1)``, ``z0 = r cos(2 pi u2)``, ``z1 = r sin(2 pi u2)``),
  uniform U(-1, 1) draws are ``2u - 1``;
* values are scaled by the standard deviation, cast to float32, then rounded
  to bf16 or fp16 with round-to-nearest-even (fp32 inputs keep the float32).

The attention workloads below are the shapes the FlashAttention forward
pass is measured and checked on (head dims 64 and 128, bf16 and fp16,
causal and not, one ragged length).  The row-softmax workloads are matrices
of attention-score-like rows (N(0, 3^2) values): a bf16 score block, fp32
rows too long for registers, and fp16 rows of odd length.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "x": 3, "a": 4, "w": 5, "bias": 6}


@dataclass(frozen=True)
class Dist:
    """A value distribution: ``kind`` is "normal" (mean 0) or "uniform" (symmetric)."""

    kind: str
    scale: float  # standard deviation for "normal", half-width for "uniform"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp16"
    causal: tuple       # which masks the workload is run with
    q: Dist
    k: Dist
    v: Dist
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def describe(self) -> str:
        return f"B={self.B},H={self.H},N={self.N},d={self.d},{self.dtype}"


N01 = Dist("normal", 1.0)
N03 = Dist("normal", 3.0)
U11 = Dist("uniform", 1.0)

WORKLOADS = {
    # small correctness case the CPU oracle finishes in well under a second
    "small": Workload("small", 1, 2, 256, 64, "fp16", (False,), N01, N01, N01),
    # mid-size, run both with and without the causal mask (shared inputs)
    "mid": Workload("mid", 4, 16, 1024, 64, "bf16", (False, True), N01, N01, N01),
    # Llama-style head, causal: the throughput target
    "llama": Workload("llama", 8, 32, 2048, 128, "bf16", (True,), N01, N01, N01),
    # long sequence, causal; Q and K with std 3 give peaky softmax rows
    "long": Workload("long", 1, 32, 8192, 128, "bf16", (True,), N03, N03, N01),
    # ragged length (not a multiple of any tile), non-causal
    "ragged": Workload("ragged", 16, 16, 4000, 64, "fp16", (False,), U11, U11, U11),
}


def _uniform01(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """n doubles in (0, 1) from the Philox stream keyed (seed, tensor_id)."""
    bg = np.random.Philox(key=np.array([seed, tensor_id], dtype=np.uint64))
    w = bg.random_raw(n)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def draw(dist: Dist, n: int, seed: int, tensor_id: int) -> np.ndarray:
    """n float32 draws of ``dist`` (before rounding to the storage type)."""
    if dist.kind == "normal":
        m = (n + 1) // 2
        u = _uniform01(seed, tensor_id, 2 * m)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        t = 2.0 * np.pi * u2
        z = np.empty(2 * m, dtype=np.float64)
        z[0::2] = r * np.cos(t)
        z[1::2] = r * np.sin(t)
        z = z[:n] * dist.scale
    elif dist.kind == "uniform":
        z = (2.0 * _uniform01(seed, tensor_id, n) - 1.0) * dist.scale
    else:
        raise ValueError(f"unknown distribution {dist.kind!r}")
    return z.astype(np.float32)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to bf16/fp16 (nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        if not np.all(np.isfinite(x)):
            raise ValueError("only finite values are rounded")
        b = x.view(np.uint32)
        bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        return ((b + bias) >> np.uint32(16)).astype(np.uint16)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bf16/fp16 storage bits to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bf16/fp16 storage bits to float64."""
    return bits_to_f32(bits, dtype).astype(np.float64)


def make_qkv(B: int, H: int, N: int, d: int, dtype: str,
             qdist: Dist = N01, kdist: Dist = N01, vdist: Dist = N01, seed: int = 0):
    """Q, K, V as uint16 storage bits, each [B, H, N, d] contiguous."""
    shape = (B, H, N, d)
    n = B * H * N * d
    out = []
    for name, dist in (("q", qdist), ("k", kdist), ("v", vdist)):
        x = draw(dist, n, seed, TENSOR_IDS[name])
        out.append(round_bits(x, dtype).reshape(shape))
    return tuple(out)


def make_workload(w: Workload):
    """Q, K, V storage bits for a named workload."""
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.q, w.k, w.v, w.seed)


def to_torch(bits: np.ndarray, dtype: str, device="cpu"):
    """Storage bits -> torch tensor of dtype bfloat16/float16 (same bits)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device) if device != "cpu" else t


@dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    dtype: str          # "fp32", "bf16" or "fp16"
    dist: Dist
    seed: int = 0

    def describe(self) -> str:
        return f"rows={self.rows},cols={self.cols},{self.dtype}"

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2


SOFTMAX_WORKLOADS = {
    # the score matrices of 16 heads for a 2048-token sequence (16 * 2048 rows of 2048 keys), bf16
    "scores": SoftmaxWorkload("scores", 32768, 2048, "bf16", N03),
    # fp32 rows of 256 KiB: longer than a wave's registers
    "wide": SoftmaxWorkload("wide", 512, 65536, "fp32", N03),
    # fp16 rows of odd length: rows start at every 2-byte offset within 16 bytes
    "odd": SoftmaxWorkload("odd", 32768, 1001, "fp16", N03),
}


def make_softmax_input(rows: int, cols: int, dtype: str, dist: Dist = N03, seed: int = 0) -> np.ndarray:
    """[rows, cols] input: float32 values for "fp32", else uint16 storage bits."""
    x = draw(dist, rows * cols, seed, TENSOR_IDS["x"]).reshape(rows, cols)
    return x if dtype == "fp32" else round_bits(x, dtype).reshape(rows, cols)


def make_softmax_workload(w: SoftmaxWorkload) -> np.ndarray:
    return make_softmax_input(w.rows, w.cols, w.dtype, w.dist, w.seed)


def softmax_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a softmax input (float32 values or 16-bit bits) to float64."""
    return np.asarray(x, dtype=np.float64) if dtype == "fp32" else bits_to_f64(x, dtype)


def softmax_to_torch(x: np.ndarray, dtype: str, device="cpu"):
    """Softmax input -> torch tensor of the matching dtype (same values)."""
    import torch

    if dtype == "fp32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(device) if device != "cpu" else t
    return to_torch(x, dtype, device)


@dataclass(frozen=True)
class GemmWorkload:
    """C = GELU(A W^T + b): A [M, K] ~ N(0, 1), W [N, K] ~ N(0, 1/K) (the
    scale of a linear layer's initialisation, so A W^T is of order 1 and
    GELU sees both signs), b [N] ~ U(-1, 1), A and W rounded to bf16."""
    name: str
    M: int
    N: int
    K: int
    seed: int = 0

    def describe(self) -> str:
        return f"M={self.M},N={self.N},K={self.K},bf16"

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


GEMM_WORKLOADS = {
    # the up-projection of a transformer MLP for the attention workload's tokens:
    # 8 x 2048 tokens, hidden 4096 (32 heads of 128), 4x expansion
    "mlp": GemmWorkload("mlp", 16384, 16384, 4096),
    # ragged in every dimension: several tiles, partial tiles, a K tail
    "ragged": GemmWorkload("ragged", 1000, 776, 328),
    "small": GemmWorkload("small", 300, 264, 200),
}


def make_gemm_inputs(M: int, N: int, K: int, seed: int = 0):
    """A, W as uint16 bf16 bits and the fp32 bias, for C = GELU(A W^T + b)."""
    a = round_bits(draw(N01, M * K, seed, TENSOR_IDS["a"]).reshape(M, K), "bf16")
    w = round_bits(draw(Dist("normal", float(K) ** -0.5), N * K, seed, TENSOR_IDS["w"]).reshape(N, K), "bf16")
    b = draw(Dist("uniform", 1.0), N, seed, TENSOR_IDS["bias"]).astype(np.float32)
    return a, w, b


def make_gemm_workload(w: GemmWorkload):
    return make_gemm_inputs(w.M, w.N, w.K, w.seed)
