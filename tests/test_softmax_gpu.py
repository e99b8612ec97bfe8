"""GPU parity of the row-wise softmax kernel (C ABI ``softmax_rows``) against
the fp64 oracle (oracle/softmax.py) on seeded inputs.

Tolerance: the kernel computes in fp32 and rounds the output to the input
type once.  Rounding to nearest costs up to half an ulp, which relative to
the value is at most 2^-8 for bf16 (8 significant bits: the bound is reached
just above a power of two) and 2^-11 for fp16; the fp32 computation before
it is accurate to a few 1e-6 relative (exponent arguments up to ~400 carry
~1e-5 of fp32 rounding), and rounding can carry that error across a
rounding midpoint.  So |y - y_ref| <= rel * |y_ref| + abs with rel = 5e-5 +
the half-ulp bound (0 for fp32).  abs covers the smallest outputs: the
hardware base-2 exponential flushes results below 2^-126 to zero (fp32 and
bf16 share that exponent range), and fp16 outputs below 2^-14 are subnormal
with a spacing of 2^-24.  Row sums must be 1 within rel plus abs times the
row length.
"""

import numpy as np
import pytest

from oracle import softmax_rows_ref
from tiled_tensor_core_amd import synth
from parity import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TOL = {"fp32": (5e-5, 2.0 ** -126), "bf16": (2.0 ** -8 + 5e-5, 2.0 ** -126), "fp16": (2.0 ** -11 + 5e-5, 2.0 ** -24)}


def _to_f64(t, dtype):
    import torch

    if dtype == "fp32":
        return t.cpu().numpy().astype(np.float64)
    bits = t.cpu().view(torch.int16).numpy().view(np.uint16)
    return synth.bits_to_f64(bits, dtype)


def run_gpu(x, dtype, inplace=False):
    """Run the kernel on input x (host array); returns the output as float64."""
    from tiled_tensor_core_amd import attn

    xt = synth.softmax_to_torch(x, dtype, "cuda")
    if inplace:
        attn.softmax_rows(xt, xt, xt.shape[0], xt.shape[1])
        yt = xt
    else:
        yt = attn.softmax(xt)
    import torch

    torch.cuda.synchronize()
    return _to_f64(yt, dtype)


def check(y, ref, dtype, tag):
    rel, ab = TOL[dtype]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(y), np.isnan(ref)), f"{tag}: NaN pattern differs"
    err = np.abs(y[fin] - ref[fin])
    bound = rel * np.abs(ref[fin]) + ab
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    print(f"[softmax parity] {tag}: max err/bound {worst:.3f}, max abs err {float(err.max()) if err.size else 0:.3e}",
          flush=True)
    assert np.all(err <= bound), f"{tag}: worst err/bound {worst}"
    rows_ok = np.all(np.isfinite(ref), axis=1)
    if np.any(rows_ok):
        sums = y[rows_ok].sum(axis=1)
        assert np.all(np.abs(sums - 1.0) <= rel * 1.0 + ab * y.shape[1] + 1e-6), f"{tag}: row sums {sums}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("rows,cols", [
    (1, 1), (3, 7), (5, 8), (2, 4), (64, 512), (33, 1000), (17, 2048), (9, 4096), (7, 8192),
    (3, 8200), (4, 12345), (2, 40000), (2, 65536), (2, 65544), (3, 70000), (1, 300000),
])
def test_shapes(dtype, rows, cols):
    x = synth.make_softmax_input(rows, cols, dtype, seed=rows * 7919 + cols)
    y = run_gpu(x, dtype)
    check(y, softmax_rows_ref(synth.softmax_to_f64(x, dtype)), dtype, f"{dtype} {rows}x{cols}")


@pytest.mark.parametrize("i", range(16))
def test_random_shapes(i):
    """Seeded random row counts (1-300), widths (1-20000, every alignment),
    dtypes and value spreads (std 0.5-8)."""
    rng = np.random.default_rng(5000 + i)
    rows = int(rng.integers(1, 301))
    cols = int(rng.integers(1, 20001))
    dtype = str(rng.choice(["fp32", "bf16", "fp16"]))
    std = float(rng.choice([0.5, 1.0, 3.0, 8.0]))
    x = synth.make_softmax_input(rows, cols, dtype, dist=synth.Dist("normal", std), seed=6000 + i)
    y = run_gpu(x, dtype)
    check(y, softmax_rows_ref(synth.softmax_to_f64(x, dtype)), dtype, f"case {i}: {dtype} {rows}x{cols} std {std}")


ODD_COLS = {  # byte lengths that are not multiples of 16; the last ones pass 16 KiB (element-wise path)
    "fp16": [1, 3, 7, 9, 15, 17, 63, 65, 129, 513, 1001, 1023, 2047, 4095, 8191, 8193, 12345],
    "bf16": [1, 5, 8, 17, 255, 1001, 2049, 8191, 8193],
    "fp32": [1, 2, 3, 5, 6, 7, 9, 255, 257, 1001, 1022, 2049, 4095, 4097, 4098],
}


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_odd_widths_every_alignment(dtype):
    """Rows whose byte length is not a multiple of 16: with 19 rows the row
    starts run through every element offset within 16 bytes, so the head
    (before the first 16-byte boundary), the aligned interior and the tail
    take every split, including rows shorter than 16 bytes that hold no
    interior at all."""
    for cols in ODD_COLS[dtype]:
        x = synth.make_softmax_input(19, cols, dtype, seed=cols + 101)
        y = run_gpu(x, dtype)
        check(y, softmax_rows_ref(synth.softmax_to_f64(x, dtype)), dtype, f"odd {dtype} 19x{cols}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_in_place(dtype):
    x = synth.make_softmax_input(10, 3000, dtype, seed=5)
    y = run_gpu(x, dtype, inplace=True)
    check(y, softmax_rows_ref(synth.softmax_to_f64(x, dtype)), dtype, f"in place {dtype}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("cols", [64, 1000, 1001, 9001, 20000, 70000])
def test_minus_inf_and_nan_rows(dtype, cols):
    """-inf entries weigh 0; an all -inf row and a row holding NaN come out NaN."""
    x = synth.softmax_to_f64(synth.make_softmax_input(6, cols, dtype, seed=cols), dtype).astype(np.float32)
    x[0, ::3] = -np.inf
    x[1, :] = -np.inf
    x[2, cols // 2] = np.nan
    x[3, 1:] = -np.inf
    if dtype == "bf16":
        bits = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # exact: x holds bf16 values
        xin, ref_in = bits, synth.bits_to_f64(bits, "bf16")
    else:
        xin, ref_in = x, x.astype(np.float64)
    y = run_gpu(xin, dtype)
    ref = softmax_rows_ref(ref_in)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    assert np.all(y[0, ::3] == 0.0)
    assert abs(y[3, 0] - 1.0) <= 1e-6 and np.all(y[3, 1:] == 0.0)
    check(y, ref, dtype, f"-inf/NaN rows {dtype} cols={cols}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("cols", [1554, 2048, 9001, 20000, 70000])
def test_large_magnitudes(dtype, cols):
    """Values of size ~1e4 on every path (odd byte lengths in registers and
    element-wise, one wave per row, one workgroup per row, segments):
    the maximum shift keeps every exponent finite, and the rounding of the
    scaled maximum must cancel between numerators and denominator (else the
    relative error reaches ulp(1e4 * log2 e) ~ 1e-3)."""
    x = (synth.make_softmax_input(8, cols, "fp32", seed=3) * 3000.0).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bits(x, "bf16")
    y = run_gpu(x, dtype)
    ref = softmax_rows_ref(synth.softmax_to_f64(x, dtype))
    assert np.all(np.isfinite(y))
    assert np.array_equal(np.argmax(y, axis=1), np.argmax(ref, axis=1))
    check(y, ref, dtype, f"large magnitudes {dtype} cols={cols}")


@pytest.mark.slow
@pytest.mark.parametrize("name", list(synth.SOFTMAX_WORKLOADS))
def test_workloads_sampled(name):
    """The measured workloads, checked on sampled rows (plus first and last)."""
    w = synth.SOFTMAX_WORKLOADS[name]
    x = synth.make_softmax_workload(w)
    y = run_gpu(x, w.dtype)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, w.rows - 1], rng.integers(0, w.rows, 64)]))
    ref = softmax_rows_ref(synth.softmax_to_f64(x[rows], w.dtype))
    check(y[rows], ref, w.dtype, f"workload {name} {w.describe()}")
    assert np.all(np.isfinite(y))
