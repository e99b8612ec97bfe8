"""GPU parity of the GEMM kernel with its fused epilogue (C ABI ``gemm_bf16``)
against the fp64 oracle (oracle/gemm.py) on seeded inputs.

Tolerance, per element: |c - c_ref| <= 2^-8 |c_ref| + (1 + 2^-8) * d with
d = 1.13 * 6 sqrt(K) 2^-24 S + 5e-7 (1 + S) and S = sum_k |a_k w_k| + |b|.
The output is the kernel's fp32 value g = c_ref + e rounded once to bf16;
rounding to nearest costs up to half an ulp, at most 2^-8 |g| (bf16 has 8
significant bits; the bound is reached just above a power of two), so
|c - c_ref| <= 2^-8 |c_ref| + (1 + 2^-8) |e|.  The fp32 error e has two
parts: accumulation, bounded with overwhelming probability by
lambda sqrt(K) u S (Higham and Mary; lambda = 6, u = 2^-24) times the
largest slope of GELU (1.13); and the Abramowitz-Stegun erfc inside the
kernel's GELU, within 4.3e-7 + 0.75e-7 |z| of the exact GELU, |z| <= S.
At the measured sizes d is a few 1e-4 against outputs of order 1.
"""

import numpy as np
import pytest

from oracle import EPI_BIAS, EPI_BIAS_GELU, EPI_NONE, gemm_ref
from tiled_tensor_core_amd import synth
from parity import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _run(a_bits, w_bits, bias, epi):
    import torch

    from tiled_tensor_core_amd import attn

    a = synth.to_torch(a_bits, "bf16", "cuda")
    w = synth.to_torch(w_bits, "bf16", "cuda")
    b = torch.from_numpy(bias).cuda() if epi != EPI_NONE else None
    c = attn.gemm(a, w, b, epilogue=epi)
    torch.cuda.synchronize()
    return synth.bits_to_f64(c.cpu().view(torch.int16).numpy().view(np.uint16), "bf16")


def _check(c, a64, w64, bias, epi, tag, rows=None):
    ref = gemm_ref(a64, w64, bias, epi)
    S = np.abs(a64) @ np.abs(w64).T + (np.abs(bias)[None, :] if epi != EPI_NONE else 0.0)
    K = a64.shape[1]
    d = 1.13 * 6.0 * np.sqrt(K) * 2.0 ** -24 * S + 5e-7 * (1.0 + S)
    bound = 2.0 ** -8 * np.abs(ref) + (1.0 + 2.0 ** -8) * d
    err = np.abs(c - ref)
    worst = float(np.max(err / bound))
    print(f"[gemm parity] {tag}: max err/bound {worst:.3f}, max abs err {float(err.max()):.3e}", flush=True)
    assert np.all(np.isfinite(c)), f"{tag}: non-finite output"
    assert np.all(err <= bound), f"{tag}: worst err/bound {worst}"


SHAPES = [  # M, N, K: one partial tile; exact tiles; ragged in all three with a K tail; tiny;
    # K a multiple of 128 (loads without bound checks) with ragged M and N
    (300, 264, 200), (256, 256, 64), (512, 512, 128), (1000, 776, 328), (1, 8, 8), (17, 24, 72), (257, 8, 4104),
    (1000, 776, 256), (300, 264, 384), (33, 40, 128),
]


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_BIAS, EPI_BIAS_GELU])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_parity(M, N, K, epi):
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=M + N + K)
    c = _run(a, w, b, epi)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), epi,
           f"{M}x{N}x{K} epi={epi}")


@pytest.mark.parametrize("i", range(16))
def test_random_shapes(i):
    """Seeded random shapes: M 1-700, N and K multiples of 8 up to 704 (K a
    multiple of 128 in some draws, the path without load bound checks), and
    a random epilogue."""
    rng = np.random.default_rng(3000 + i)
    M = int(rng.integers(1, 701))
    N = 8 * int(rng.integers(1, 89))
    K = 128 * int(rng.integers(1, 6)) if rng.integers(0, 3) == 0 else 8 * int(rng.integers(1, 89))
    epi = int(rng.choice([EPI_NONE, EPI_BIAS, EPI_BIAS_GELU]))
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=4000 + i)
    c = _run(a, w, b, epi)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), epi,
           f"case {i}: {M}x{N}x{K} epi={epi}")


@pytest.mark.parametrize("M,N,K", [(8, 8, 4194296), (5, 8, 4194176), (8, 4194296, 8)])
def test_largest_dimensions(M, N, K):
    """N and K at the boundary's limit (4194296: 256 rows of them in bf16 fit
    the 2^31-byte range of a tile's buffer) or the largest multiple of 128
    below it (the path without load bound checks): every element against the
    oracle."""
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=K + N)
    c = _run(a, w, b, EPI_BIAS_GELU)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), EPI_BIAS_GELU,
           f"{M}x{N}x{K} at the size limit")


def test_many_tiles_every_element():
    """342 tiles of 256 x 256 (one full window of 256 concurrently running
    tiles and a partial one, ragged in M and N): every element against the
    oracle, so a tile computed twice or never would show."""
    M, N, K = 17 * 256 + 5, 19 * 256 - 8, 128   # N a multiple of 8
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=21)
    c = _run(a, w, b, EPI_BIAS_GELU)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), EPI_BIAS_GELU,
           f"{M}x{N}x{K} every element")


@pytest.mark.parametrize("M,N,K", [(2049, 4088, 1024), (1000, 776, 384)])
def test_ragged_tiles_without_k_checks(M, N, K):
    """K a multiple of 128 (loads without k checks), M and N ragged: the
    last tile row holds one row of A (2049 = 8 * 256 + 1), the last tile
    column 248 rows of W, over 128 tiles of 256 x 256 (the main kernel) and,
    second shape, under (the small-problem kernel).  The rows of a piece past
    M or N must fall outside the tile's buffer range (the range check covers
    the lane offset only); every element against the oracle."""
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=M + K)
    c = _run(a, w, b, EPI_BIAS_GELU)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), EPI_BIAS_GELU,
           f"{M}x{N}x{K} ragged, no k checks")


@pytest.mark.parametrize("K", [384, 320, 64, 200, 72])
def test_four_wave_kernel_every_element(K):
    """272 tiles of 256 x 256, ragged in M and N.  K = 384 (an even number
    of 64-wide slices: the 4-wave kernel's loop runs twice, then its tail),
    320 and 64 (an odd number, rounded up by a slice of zeros) run the 4-wave
    kernel, which runs the MLP workload; K = 200 and 72 (not multiples of 64)
    the 8-wave kernel.  Every element against the oracle."""
    M, N = 16 * 256 + 3, 16 * 256 - 8
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=31 + K)
    c = _run(a, w, b, EPI_BIAS_GELU)
    _check(c, synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64), EPI_BIAS_GELU,
           f"{M}x{N}x{K} every element, 4-wave kernel")


def test_gelu_range_and_large_values():
    """Pre-activations from -40 to 40 (scaled weights): both GELU tails and the
    region around 0, where GELU bends, are exercised."""
    M, N, K = 256, 264, 256
    a, w, b = synth.make_gemm_inputs(M, N, K, seed=9)
    w = synth.round_bits(synth.bits_to_f32(w, "bf16") * 16.0, "bf16")   # |z| up to ~40
    b = (b * 4.0).astype(np.float32)
    c = _run(a, w, b, EPI_BIAS_GELU)
    a64, w64 = synth.bits_to_f64(a, "bf16"), synth.bits_to_f64(w, "bf16")
    z = a64 @ w64.T + b
    assert z.min() < -20 and z.max() > 20
    _check(c, a64, w64, b.astype(np.float64), EPI_BIAS_GELU, "wide pre-activations")


@pytest.mark.slow
def test_mlp_workload_sampled_rows():
    """The measured workload at full size, checked on sampled rows (first,
    last and 30 random) of C against the oracle."""
    import torch

    from tiled_tensor_core_amd import attn

    wl = synth.GEMM_WORKLOADS["mlp"]
    a, w, b = synth.make_gemm_workload(wl)
    at = synth.to_torch(a, "bf16", "cuda")
    wt = synth.to_torch(w, "bf16", "cuda")
    c = attn.gemm(at, wt, torch.from_numpy(b).cuda(), epilogue=EPI_BIAS_GELU)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.integers(0, wl.M, 30)]))
    ct = c[torch.from_numpy(rows).cuda()].cpu()
    cr = synth.bits_to_f64(ct.view(torch.int16).numpy().view(np.uint16), "bf16")
    _check(cr, synth.bits_to_f64(a[rows], "bf16"), synth.bits_to_f64(w, "bf16"), b.astype(np.float64),
           EPI_BIAS_GELU, f"mlp {wl.describe()} sampled rows")
    assert bool(torch.isfinite(c.float()).all())


def test_rejects_bad_arguments_before_launch():
    import torch

    from tiled_tensor_core_amd import attn

    a = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.gemm_bf16(a, w, None, c, 4, 8, 16, attn.GEMM_EPI_BIAS)
    assert e.value.code == 1
    # K = 12 is no multiple of 8: tensors sized for it pass the binding's
    # checks, and the C ABI rejects the shape
    a12 = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    w12 = torch.zeros((8, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.gemm_bf16(a12, w12, None, c, 4, 8, 12, attn.GEMM_EPI_NONE)
    assert e.value.code == 2
