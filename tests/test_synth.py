"""CPU tests of the seeded input generator (no attention arithmetic here)."""

import numpy as np
import pytest

from tiled_tensor_core_amd import synth


def test_deterministic_and_streams_distinct():
    a = synth.make_qkv(1, 2, 64, 16, "bf16", seed=0)
    b = synth.make_qkv(1, 2, 64, 16, "bf16", seed=0)
    c = synth.make_qkv(1, 2, 64, 16, "bf16", seed=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert not np.array_equal(a[0], a[1]) and not np.array_equal(a[1], a[2])


def test_prefix_stable():
    """A tensor's draws depend only on (seed, tensor id) and position, so a
    bigger tensor starts with the smaller one's values."""
    x = synth.draw(synth.N01, 1000, 0, 2)
    y = synth.draw(synth.N01, 101, 0, 2)
    assert np.array_equal(x[:101], y)


@pytest.mark.parametrize("dist,mean,std", [(synth.N01, 0.0, 1.0), (synth.N03, 0.0, 3.0),
                                           (synth.U11, 0.0, 1 / np.sqrt(3))])
def test_moments(dist, mean, std):
    x = synth.draw(dist, 400_000, 0, 0).astype(np.float64)
    assert abs(x.mean() - mean) < 0.01 * max(std, 1)
    assert abs(x.std() - std) < 0.01 * std
    if dist.kind == "uniform":
        assert x.min() > -1 and x.max() < 1


def test_bf16_round_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 2.0 ** 127,
                  1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    bits = synth.round_bits(f, "bf16")
    back = synth.bits_to_f32(bits, "bf16")
    # ties go to even: 1+2^-8 is halfway between 1 and 1+2^-7 -> 1
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> 1+2^-6 (even mantissa)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 2.0 ** 127, 1.0 + 2 ** -7],
                    dtype=np.float32)
    assert np.array_equal(back[:6], want[:6])
    assert back[6] == np.float32(1.0 + 2 ** -7)
    # agrees with torch's own conversion
    import torch
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, bits)


def test_fp16_round_and_widen():
    f = np.array([0.1, -1.5, 65504.0, 1e-6], dtype=np.float32)
    bits = synth.round_bits(f, "fp16")
    assert np.array_equal(synth.bits_to_f32(bits, "fp16"), f.astype(np.float16).astype(np.float32))


def test_workloads_shapes():
    w = synth.WORKLOADS["small"]
    q, k, v = synth.make_workload(w)
    assert q.shape == (1, 2, 256, 64) and q.dtype == np.uint16
    assert synth.WORKLOADS["ragged"].N % 64 != 0
    assert abs(synth.WORKLOADS["llama"].scale - 1 / np.sqrt(128)) < 1e-15


def test_to_torch_same_bits():
    import torch
    q, _, _ = synth.make_qkv(1, 1, 8, 16, "fp16", seed=3)
    t = synth.to_torch(q, "fp16")
    assert t.dtype == torch.float16
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), q)


def test_softmax_input_deterministic_and_typed():
    a = synth.make_softmax_input(5, 33, "bf16", seed=4)
    b = synth.make_softmax_input(5, 33, "bf16", seed=4)
    assert a.dtype == np.uint16 and a.shape == (5, 33)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.make_softmax_input(5, 33, "bf16", seed=5))
    f = synth.make_softmax_input(5, 33, "fp32", seed=4)
    assert f.dtype == np.float32
    # the 16-bit input is the fp32 draw rounded to nearest even
    assert np.array_equal(a, synth.round_bits(f, "bf16"))
    # the softmax stream is not the Q/K/V streams
    q = synth.draw(synth.N03, 5 * 33, 4, synth.TENSOR_IDS["q"])
    assert not np.array_equal(q.reshape(5, 33), f)


def test_softmax_widening_is_exact():
    bits = synth.make_softmax_input(4, 40, "fp16", seed=1)
    x64 = synth.softmax_to_f64(bits, "fp16")
    assert np.array_equal(x64.astype(np.float16).view(np.uint16), bits)
    t = synth.softmax_to_torch(bits, "fp16")
    assert np.array_equal(t.view(__import__("torch").int16).numpy().view(np.uint16), bits)
    f = synth.make_softmax_input(3, 7, "fp32")
    assert np.array_equal(synth.softmax_to_f64(f, "fp32"), f.astype(np.float64))


def test_softmax_workloads():
    for name, w in synth.SOFTMAX_WORKLOADS.items():
        assert w.name == name and w.rows > 0 and w.cols > 0
        assert w.elem_bytes == (4 if w.dtype == "fp32" else 2)
    # the three kernel paths: rows within one wave's registers, rows of a
    # workgroup, and rows whose byte length is not a multiple of 16
    sizes = {n: w.cols * w.elem_bytes for n, w in synth.SOFTMAX_WORKLOADS.items()}
    assert sizes["scores"] <= 16384 and sizes["scores"] % 16 == 0
    assert 16384 < sizes["wide"] <= 262144 and sizes["wide"] % 16 == 0
    assert sizes["odd"] % 16 != 0


def test_gemm_inputs():
    a, w, b = synth.make_gemm_inputs(6, 16, 64, seed=2)
    a2, w2, b2 = synth.make_gemm_inputs(6, 16, 64, seed=2)
    assert a.dtype == np.uint16 and a.shape == (6, 64) and w.shape == (16, 64) and b.shape == (16,)
    assert b.dtype == np.float32 and np.array_equal(a, a2) and np.array_equal(w, w2) and np.array_equal(b, b2)
    # W ~ N(0, 1/K): a linear layer's initialisation scale; b ~ U(-1, 1)
    wl = synth.bits_to_f64(synth.make_gemm_inputs(4, 256, 1024, seed=3)[1], "bf16")
    assert abs(wl.std() * np.sqrt(1024) - 1.0) < 0.02
    assert np.all(np.abs(b) <= 1.0)
    for name, g in synth.GEMM_WORKLOADS.items():
        assert g.name == name and g.N % 8 == 0 and g.K % 8 == 0 and g.flops() == 2.0 * g.M * g.N * g.K
