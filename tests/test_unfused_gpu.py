"""GPU parity of the un-fused attention path (scores in device memory, row
softmax in place, then P V) against the fp64 oracle, through the C ABI.

O and LSE meet the same bar as the fused kernel (O max-abs <= 1e-2, relative
Frobenius <= 5e-3, LSE max-abs <= 1e-3).  The probability matrix the path
leaves in its workspace is compared entry by entry with the oracle's
attention_probs: the scores are fp32 sums of products of 16-bit inputs, and
the fp32 softmax of the row-softmax kernel (relative error about 5e-5) turns
a score error e into a relative error of about e, so the bound is
|P - P_ref| <= 1e-4 |P_ref| + 1e-7.
"""

import numpy as np
import pytest

from oracle import attention_probs, attention_ref
from parity import assert_close, gpu_available
from tiled_tensor_core_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _run(qb, kb, vb, dtype, causal, scale):
    import torch

    from tiled_tensor_core_amd import attn

    q, k, v = (synth.to_torch(x, dtype, "cuda") for x in (qb, kb, vb))
    B, H, N, d = q.shape
    need = attn.attn_unfused_workspace_bytes(B, H, N)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    attn.attn_fwd_unfused(q, k, v, o, lse, ws, need, B, H, N, d, int(causal), scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), ws.view(B, H, N, N).cpu().numpy()


def _check(qb, kb, vb, dtype, causal, scale, tag, probs=True):
    o, lse, p = _run(qb, kb, vb, dtype, causal, scale)
    q64, k64, v64 = (synth.bits_to_f64(x, dtype) for x in (qb, kb, vb))
    o_ref, l_ref = attention_ref(q64, k64, v64, causal, scale)
    assert_close(o, lse, o_ref, l_ref, tag)
    if probs:
        p_ref = attention_probs(q64, k64, causal, scale)
        err = np.abs(p - p_ref) / (1e-4 * np.abs(p_ref) + 1e-7)
        print(f"[probs] {tag} worst error / bound {err.max():.3f}", flush=True)
        assert err.max() <= 1.0, tag
        if causal:
            assert np.all(p[..., np.triu(np.ones(p.shape[-2:], dtype=bool), 1)] == 0.0)


def test_small_workload():
    w = synth.WORKLOADS["small"]
    q, k, v = synth.make_workload(w)
    for causal in (False, True):
        _check(q, k, v, w.dtype, causal, w.scale, f"unfused small causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_mid_workload(causal):
    w = synth.WORKLOADS["mid"]
    q, k, v = synth.make_workload(w)
    # the 64 x 1024^2 probability matrix is checked on the small shapes below
    _check(q, k, v, w.dtype, causal, w.scale, f"unfused mid causal={causal}", probs=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_inputs_follow_the_definition(dtype, causal):
    """As for the fused kernel: a NaN in one key row reaches exactly the query
    rows that see it, a NaN in one query row only that row."""
    B, H, N, d = 1, 2, 300, 64
    q, k, v = synth.make_qkv(B, H, N, d, dtype, seed=11 + int(causal))
    nan_bits = np.uint16(0x7FC0 if dtype == "bf16" else 0x7E00)
    k[0, 0, 137, :] = nan_bits
    q[0, 1, 200, 5] = nan_bits
    o, lse, _ = _run(q, k, v, dtype, causal, 0.125)
    q64, k64, v64 = (synth.bits_to_f64(x, dtype) for x in (q, k, v))
    o_ref, l_ref = attention_ref(q64, k64, v64, causal, 0.125)
    nan_rows = np.isnan(l_ref)
    assert nan_rows.any() and not nan_rows.all()
    assert np.array_equal(np.isnan(lse), nan_rows), "LSE NaN rows differ from the oracle's"
    assert np.array_equal(np.isnan(o).any(axis=-1), nan_rows), "O NaN rows differ from the oracle's"
    assert np.array_equal(np.isnan(o).all(axis=-1), nan_rows), "a NaN row of O is only partly NaN"
    fin = ~nan_rows
    assert_close(o[fin][None], lse[fin][None], o_ref[fin][None], l_ref[fin][None],
                 tag=f"unfused finite rows {dtype} causal={causal}")


@pytest.mark.parametrize("i", range(8))
def test_random_configurations(i):
    """Seeded random batch, heads, lengths (1-400), head dims, dtypes, masks,
    Q/K spreads and signed scales; O, LSE and the probability matrix."""
    rng = np.random.default_rng(7000 + i)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    N = int(rng.integers(1, 401))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    causal = bool(rng.integers(0, 2))
    std = float(rng.choice([0.5, 1.0, 2.0]))
    scale = float(rng.choice([0.5, 1.0, -1.0])) / float(np.sqrt(d))
    qk = synth.Dist("normal", std)
    q, k, v = synth.make_qkv(B, H, N, d, dtype, qk, qk, synth.Dist("normal", 1.0), seed=8000 + i)
    _check(q, k, v, dtype, causal, scale,
           f"unfused case {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} std {std} scale {scale:.4g}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 33, 64, 65, 127, 129, 200, 257])
def test_shapes(dtype, d, causal, N):
    dist = synth.Dist("normal", 1.0)
    q, k, v = synth.make_qkv(1, 3, N, d, dtype, dist, dist, dist, seed=N + 7)
    _check(q, k, v, dtype, causal, 1 / np.sqrt(d), f"unfused {dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
def test_scales(scale):
    dist = synth.Dist("normal", 1.0)
    q, k, v = synth.make_qkv(2, 2, 150, 64, "bf16", dist, dist, dist, seed=5)
    for causal in (False, True):
        _check(q, k, v, "bf16", causal, scale, f"unfused scale={scale} causal={causal}")


def test_matches_fused_path():
    """The two HIP paths agree with each other as they do with the oracle
    (each within the tolerance, so within twice it of each other)."""
    import torch

    from tiled_tensor_core_amd import attn

    dist = synth.Dist("normal", 1.0)
    qb, kb, vb = synth.make_qkv(2, 4, 300, 128, "bf16", dist, dist, dist, seed=9)
    q, k, v = (synth.to_torch(x, "bf16", "cuda") for x in (qb, kb, vb))
    for causal in (False, True):
        o1, l1 = attn.fwd(q, k, v, causal, 128 ** -0.5)
        o2, l2 = attn.fwd_unfused(q, k, v, causal, 128 ** -0.5)
        torch.cuda.synchronize()
        assert float((o1 - o2).abs().max()) <= 2e-2
        assert float((l1 - l2).abs().max()) <= 2e-3
