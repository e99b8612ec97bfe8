"""GPU parity tests: the HIP path (through the C ABI binding) against the fp64
oracle, element by element, on the same seeded inputs.

Tolerances (in tests/parity.py): O max-abs <= 1e-2 and relative Frobenius
<= 5e-3, LSE max-abs <= 1e-3.  The five measured workloads run at their full
sizes in the launch configuration the benchmark times; the two largest are
checked on whole sampled heads plus sampled rows of every head.
"""

import numpy as np
import pytest

from oracle import attention_ref
from parity import assert_close, full_check, gpu_available, run_hip, sampled_check
from tiled_tensor_core_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

W = synth.WORKLOADS


def _bits(shape, dtype, seed, std=1.0, kind="normal"):
    B, H, N, d = shape
    dist = synth.Dist(kind, std)
    return synth.make_qkv(B, H, N, d, dtype, dist, dist, dist, seed=seed)


# ---- the five workloads --------------------------------------------------------

def test_workload_small():
    w = W["small"]
    q, k, v = synth.make_workload(w)
    full_check(q, k, v, w.dtype, False, w.scale, tag="small non-causal")


@pytest.mark.parametrize("causal", [False, True])
def test_workload_mid(causal):
    w = W["mid"]
    q, k, v = synth.make_workload(w)
    full_check(q, k, v, w.dtype, causal, w.scale, tag=f"mid causal={causal}")


@pytest.mark.slow
@pytest.mark.parametrize("name,full_heads,rows", [
    ("llama", {0, 37, 128, 255}, 24),
    ("long", {0, 31}, 48),
    ("ragged", {0, 100, 255}, 24),
])
def test_workload_full_size(name, full_heads, rows):
    w = W[name]
    q, k, v = synth.make_workload(w)
    for causal in w.causal:
        o, lse = run_hip(q, k, v, w.dtype, causal, w.scale)
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        sampled_check(q, k, v, w.dtype, causal, w.scale, o, lse, full_heads, rows,
                      tag=f"{name} causal={causal}")


# ---- shapes: tails on both edges, tiny and ragged lengths ----------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 64, 65, 127, 129, 200, 257, 383])
def test_shapes(dtype, d, causal, N):
    q, k, v = _bits((1, 3, N, d), dtype, seed=N)
    full_check(q, k, v, dtype, causal, 1 / np.sqrt(d), tag=f"{dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("B,H", [(1, 1), (3, 5), (2, 8), (16, 1)])
def test_batch_head_mapping(B, H):
    """Head counts that are and are not multiples of 8 (XCD-aware mapping on/off)."""
    q, k, v = _bits((B, H, 150, 64), "bf16", seed=B * 10 + H)
    for causal in (False, True):
        full_check(q, k, v, "bf16", causal, 0.125, tag=f"B={B} H={H} causal={causal}")


# ---- scale and value edge cases -----------------------------------------------

@pytest.mark.parametrize("scale", [-0.125, 0.0, 1e-30, 2.0, -1.5])
def test_scale_values(scale):
    q, k, v = _bits((1, 2, 130, 64), "bf16", seed=7)
    for causal in (False, True):
        full_check(q, k, v, "bf16", causal, scale, tag=f"scale={scale} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_peaky_rows(dtype):
    """Std-4 Q and K at d=128: logits with std ~16 make the running maximum
    jump between tiles and stress the rescale."""
    B, H, N, d = 1, 4, 700, 128
    q, k, _ = _bits((B, H, N, d), dtype, seed=11, std=4.0)
    _, _, v = _bits((B, H, N, d), dtype, seed=12)
    for causal in (False, True):
        full_check(q, k, v, dtype, causal, 1 / np.sqrt(d), tag=f"peaky {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_dominant_key_below_the_rescale_margin(d):
    """A key in the second tile outweighs the first tile's maximum by a factor
    p = 2.0077 (under the bf16 kernel's 2^2 margin, so the reference maximum
    stays at the first tile).  bf16 rounds that P to 2.0, 0.38 % low.  Keys 0
    and 64 share one large value row (|v| up to 40), so the exact O is that
    row.  If O were divided by the sum of the unrounded p, the rounding would
    pull O 0.26 % towards 0, up to 0.1: ten times the tolerance."""
    B, H, N = 1, 2, 256
    q = np.zeros((B, H, N, d), dtype=np.float32)
    q[..., 0] = 1.0
    k = np.zeros((B, H, N, d), dtype=np.float32)
    k[..., 0] = -32.0          # p = exp(-22.3) relative to key 0
    k[:, :, 0, 0] = 0.0
    k[:, :, 64, 0] = 1.0
    scale = float(np.log(2.0) + np.log1p(0.98 * 2.0 ** -8))   # key 64: p = 2 (1 + 0.98 * 2^-8)
    rng = np.random.default_rng(31)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    big = np.clip(16.0 * rng.standard_normal((B, H, d)), -40.0, 40.0).astype(np.float32)
    v[:, :, 0] = big
    v[:, :, 64] = big
    qb, kb, vb = (synth.round_bits(x, "bf16") for x in (q, k, v))
    for causal in (False, True):
        full_check(qb, kb, vb, "bf16", causal, scale, tag=f"dominant key d={d} causal={causal}")


def test_increasing_keys():
    """Scores that grow along the key axis: every tile raises the maximum."""
    B, H, N, d = 1, 1, 300, 64
    q = np.ones((B, H, N, d), dtype=np.float32)
    k = np.broadcast_to(np.linspace(-3, 3, N, dtype=np.float32)[None, None, :, None], (B, H, N, d))
    _, _, vb = _bits((B, H, N, d), "bf16", seed=3)
    qb, kb = synth.round_bits(q, "bf16"), synth.round_bits(k, "bf16")
    for causal in (False, True):
        full_check(qb, kb, vb, "bf16", causal, 0.5, tag=f"increasing keys causal={causal}")


# ---- exact properties the mathematics fixes ---------------------------------------

def test_first_causal_row_is_v0():
    B, H, N, d = 2, 2, 200, 128
    q, k, v = _bits((B, H, N, d), "bf16", seed=21)
    o, lse = run_hip(q, k, v, "bf16", True, 1 / np.sqrt(d))
    v0 = synth.bits_to_f32(v[:, :, 0], "bf16")
    np.testing.assert_allclose(o[:, :, 0].cpu().numpy(), v0, rtol=1e-6, atol=0)
    s00 = np.einsum("bhd,bhd->bh", synth.bits_to_f64(q[:, :, 0], "bf16"),
                    synth.bits_to_f64(k[:, :, 0], "bf16")) / np.sqrt(d)
    np.testing.assert_allclose(lse[:, :, 0].cpu().numpy(), s00, rtol=0, atol=1e-5)


def test_constant_v():
    B, H, N, d = 1, 2, 333, 64
    q, k, _ = _bits((B, H, N, d), "fp16", seed=22)
    c = synth.round_bits(np.random.default_rng(0).standard_normal((B, H, 1, d)).astype(np.float32), "fp16")
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    for causal in (False, True):
        o, _ = run_hip(q, k, v, "fp16", causal, 0.125)
        # P is rounded to fp16 before P.V while l sums the unrounded p, so
        # O = c * sum(round(p)) / sum(p): off by at most the fp16 unit
        # roundoff 2^-11 (plus fp32 slack)
        np.testing.assert_allclose(o.cpu().numpy(), np.broadcast_to(synth.bits_to_f32(c, "fp16"), o.shape),
                                   rtol=6e-4, atol=1e-7)


def test_equal_keys_uniform_weights():
    B, H, N, d = 1, 2, 260, 128
    q, _, v = _bits((B, H, N, d), "bf16", seed=23)
    k1 = synth.round_bits(np.random.default_rng(1).standard_normal((B, H, 1, d)).astype(np.float32), "bf16")
    k = np.broadcast_to(k1, (B, H, N, d)).copy()
    vf = synth.bits_to_f64(v, "bf16")
    for causal in (False, True):
        o, lse = run_hip(q, k, v, "bf16", causal, 1 / np.sqrt(d))
        n = np.arange(1, N + 1) if causal else np.full(N, N)
        want = np.cumsum(vf, axis=2) / n[:, None] if causal else np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        np.testing.assert_allclose(o.cpu().numpy(), want, rtol=0, atol=1e-5)
        s = np.einsum("bhnd,bhd->bhn", synth.bits_to_f64(q, "bf16"), synth.bits_to_f64(k1[:, :, 0], "bf16")) / np.sqrt(d)
        np.testing.assert_allclose(lse.cpu().numpy(), s + np.log(n), rtol=0, atol=1e-4)


# ---- memory behaviour ------------------------------------------------------------

def test_writes_every_row_and_nothing_else():
    """Outputs start NaN-poisoned inside guard bands of a sentinel value: every
    row < N must be written, no byte outside o and lse may change."""
    import torch

    from tiled_tensor_core_amd import attn

    B, H, N, d = 2, 3, 4000 // 16 + 3, 64
    qb, kb, vb = _bits((B, H, N, d), "fp16", seed=31, kind="uniform")
    q, k, v = (synth.to_torch(x, "fp16", "cuda") for x in (qb, kb, vb))
    guard = 4096
    sentinel = 12345.0
    obuf = torch.full((guard + B * H * N * d + guard,), sentinel, dtype=torch.float32, device="cuda")
    lbuf = torch.full((guard + B * H * N + guard,), sentinel, dtype=torch.float32, device="cuda")
    o = obuf[guard:guard + B * H * N * d].view(B, H, N, d)
    lse = lbuf[guard:guard + B * H * N].view(B, H, N)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    for causal in (False, True):
        attn.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, 0.125)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        assert (obuf[:guard] == sentinel).all() and (obuf[-guard:] == sentinel).all()
        assert (lbuf[:guard] == sentinel).all() and (lbuf[-guard:] == sentinel).all()
        o_ref, l_ref = attention_ref(synth.bits_to_f64(qb, "fp16"), synth.bits_to_f64(kb, "fp16"),
                                     synth.bits_to_f64(vb, "fp16"), causal, 0.125)
        assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, tag=f"guarded causal={causal}")


def test_deterministic():
    q, k, v = _bits((2, 4, 500, 128), "bf16", seed=41)
    a = run_hip(q, k, v, "bf16", True, 0.09)
    b = run_hip(q, k, v, "bf16", True, 0.09)
    assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
    assert np.array_equal(a[1].cpu().numpy(), b[1].cpu().numpy())


@pytest.mark.parametrize("entry", ["attn_fwd_bf16", "attn_fwd"])
def test_side_stream_and_entry_points(entry):
    import torch

    q, k, v = _bits((1, 8, 256, 64), "bf16", seed=51)
    ref = run_hip(q, k, v, "bf16", False, 0.125)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run_hip(q, k, v, "bf16", False, 0.125, stream=s, entry=entry)
    assert np.array_equal(ref[0].cpu().numpy(), got[0].cpu().numpy())


def test_fp16_entry_rejects_nothing_valid():
    q, k, v = _bits((1, 2, 96, 128), "fp16", seed=61)
    o, lse = run_hip(q, k, v, "fp16", True, 0.1, entry="attn_fwd_fp16")
    o_ref, l_ref = attention_ref(synth.bits_to_f64(q, "fp16"), synth.bits_to_f64(k, "fp16"),
                                 synth.bits_to_f64(v, "fp16"), True, 0.1)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, tag="fp16 entry")
