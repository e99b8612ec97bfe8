"""GPU parity tests: the HIP path (through the C ABI binding) against the fp64
oracle, element by element, on the same seeded inputs.

Tolerances (in tests/parity.py): O max-abs <= 1e-2 and relative Frobenius
<= 5e-3, LSE max-abs <= 1e-3.  The five measured workloads run at their full
sizes in the launch configuration the benchmark times, every row of every
head compared.
"""

import numpy as np
import pytest

from oracle import attention_ref
from parity import assert_close, full_check, gpu_available, run_hip, whole_check
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
@pytest.mark.parametrize("name", ["llama", "long", "ragged"])
def test_workload_full_size(name):
    """Every row of every head of the three large workloads against the
    one-shot oracle, in the launch configuration the benchmark times."""
    w = W[name]
    q, k, v = synth.make_workload(w)
    for causal in w.causal:
        print(f"[case] {name} causal={causal} {w.describe()}", flush=True)
        o, lse = run_hip(q, k, v, w.dtype, causal, w.scale)
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        whole_check(q, k, v, w.dtype, causal, w.scale, o, lse, tag=f"{name} causal={causal}")


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


@pytest.mark.parametrize("B,H,N,d,dtype", [(7, 10001, 5, 64, "bf16"), (5, 411, 130, 128, "fp16")])
def test_many_heads(B, H, N, d, dtype):
    """Far more items than resident workgroups: 70007 one-block heads (B*H
    above 2^16, not a multiple of 8, so the last group of heads is partial),
    and 2055 heads of two blocks each, the second ragged; every row of every
    head against the oracle, both masks."""
    q, k, v = _bits((B, H, N, d), dtype, seed=B + H + N)
    for causal in (False, True):
        full_check(q, k, v, dtype, causal, 1 / np.sqrt(d), tag=f"B={B} H={H} N={N} d={d} causal={causal}")


# ---- seeded random configurations ----------------------------------------------

def _random_case(i):
    """Configuration i of a fixed, seeded draw: batch, heads, a length from 1
    to 600 (most not a multiple of the 64-key tile), head dim, dtype, mask,
    the value distribution of Q and K, and the scale (a multiple of
    1/sqrt(d), negative in some cases)."""
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 6))
    N = int(rng.integers(1, 601))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    causal = bool(rng.integers(0, 2))
    kind = str(rng.choice(["normal", "uniform"]))
    std = float(rng.choice([0.5, 1.0, 2.0, 3.0]))
    scale = float(rng.choice([0.5, 1.0, 2.0, -1.0])) / float(np.sqrt(d))
    return B, H, N, d, dtype, causal, kind, std, scale


@pytest.mark.parametrize("i", range(24))
def test_random_configurations(i):
    B, H, N, d, dtype, causal, kind, std, scale = _random_case(i)
    qk = synth.Dist(kind, std)
    q, k, v = synth.make_qkv(B, H, N, d, dtype, qk, qk, synth.Dist("normal", 1.0), seed=2000 + i)
    full_check(q, k, v, dtype, causal, scale,
               tag=f"case {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} {kind}({std}) scale={scale:.4g}")


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


# The kernel moves its exponent reference only when a row outgrows it by a
# margin (2^2 in probability units for bf16, 2^8 for fp16), so the largest P
# of a row can exceed 1 and carry a 16-bit rounding error.  The cases below
# put one or several keys just under half an ulp above 2 (p = 2 (1 + 0.98 u),
# u the unit roundoff: 2^-8 for bf16, 2^-11 for fp16), so each P rounds to 2
# and is 0.98 u low, and give those keys and key 0 one large value row.  The
# exact O is that row; O divided by anything but the sum of the rounded P
# would miss it by about u |v|.
_UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def _peak_case(dtype, d, keys, vmax, seed):
    B, H, N = 1, 2, 256
    q = np.zeros((B, H, N, d), dtype=np.float32)
    q[..., 0] = 1.0
    k = np.zeros((B, H, N, d), dtype=np.float32)
    k[..., 0] = -32.0          # p = exp(-22) and less relative to key 0
    k[:, :, 0, 0] = 0.0
    for j in keys:
        k[:, :, j, 0] = 1.0
    scale = float(np.log(2.0) + np.log1p(0.98 * _UNIT_ROUNDOFF[dtype]))
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    big = np.clip(vmax / 2.5 * rng.standard_normal((B, H, d)), -vmax, vmax).astype(np.float32)
    big[..., 0] = vmax
    for j in (0, *keys):
        v[:, :, j] = big
    return (synth.round_bits(x, dtype) for x in (q, k, v)), scale


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_dominant_key_below_the_rescale_margin(dtype, d):
    """One key of the second tile at p = 2 (1 + 0.98 u) relative to the first
    tile's maximum, |v| up to 40."""
    (qb, kb, vb), scale = _peak_case(dtype, d, (64,), 40.0, 31)
    for causal, mode in ((False, 1), (True, 1), (False, 2), (True, 2)):
        m = full_check(qb, kb, vb, dtype, causal, scale, cfg={"mode": mode},
                       tag=f"dominant key {dtype} d={d} mode={mode} causal={causal}")
        # the exact O of every row that sees key 64 is the large value row:
        # far inside the tolerance, not merely within it
        assert m["o_max_abs"] <= 2e-3, m


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("keys", [(64, 65), (64, 68, 100), (70, 75, 90, 127)])
def test_tied_keys_below_the_rescale_margin(dtype, d, keys):
    """Several keys tied at a tile's maximum, all at p = 2 (1 + 0.98 u) under
    the margin, |v| = 8: in one lane, in both halves of a row's lanes
    (keys 64 and 68) and in both 32-key blocks of the tile (key 100)."""
    (qb, kb, vb), scale = _peak_case(dtype, d, keys, 8.0, 37)
    for causal, mode in ((False, 1), (True, 1), (False, 2), (True, 2)):
        m = full_check(qb, kb, vb, dtype, causal, scale, cfg={"mode": mode},
                       tag=f"tied keys {keys} {dtype} d={d} mode={mode} causal={causal}")
        assert m["o_max_abs"] <= 1e-3, m


RUNNING = {"mode": 2}     # attn_launch_cfg with the running-maximum exponent reference


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", [1, 2])
def test_increasing_keys(dtype, d, mode):
    """Scores that grow along the key axis: every tile raises the maximum.
    With the first tile's maximum as the reference the later P overflow (by
    far more than fp32's range), so in fixed-reference mode every item is
    computed again with exact row maxima; the running maximum moves every
    tile."""
    B, H, N = 1, 2, 300
    q = np.ones((B, H, N, d), dtype=np.float32)
    k = np.broadcast_to(np.linspace(-3, 3, N, dtype=np.float32)[None, None, :, None], (B, H, N, d))
    _, _, vb = _bits((B, H, N, d), dtype, seed=3)
    qb, kb = synth.round_bits(q, dtype), synth.round_bits(k, dtype)
    for causal in (False, True):
        full_check(qb, kb, vb, dtype, causal, 0.5, cfg={"mode": mode},
                   tag=f"increasing keys {dtype} d={d} mode={mode} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_recompute_inside_one_list(dtype, d):
    """One persistent workgroup works through every item of 6 heads, of which
    heads 1 and 4 (and, causal, only their later query blocks) have keys
    whose scores rise far above their first tile's: the recomputed items sit
    in the middle and at the end of the list, next to items that need none."""
    B, H, N = 1, 6, 520
    qb, kb, vb = _bits((B, H, N, d), dtype, seed=71)
    q = synth.bits_to_f32(qb, dtype)
    k = synth.bits_to_f32(kb, dtype)
    ramp = np.linspace(0.0, 12.0, N, dtype=np.float32)[:, None] * np.sign(q[0, 0, :1, :])  # grows with q_0
    for h in (1, 4):
        q[0, h] = np.abs(q[0, h]) * np.sign(q[0, 0, :1, :])
        k[0, h] = k[0, h] + ramp
    qb, kb = synth.round_bits(q, dtype), synth.round_bits(k, dtype)
    for causal in (False, True):
        for cfg in ({"n_dom": 1, "n_work": 1}, {"n_dom": 1, "n_work": 1, "mode": 2}, None):
            full_check(qb, kb, vb, dtype, causal, 1 / np.sqrt(d), cfg=cfg,
                       tag=f"recompute in one list {dtype} d={d} cfg={cfg} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 64, 129, 257, 383])
def test_shapes_running_mode(dtype, d, causal, N):
    q, k, v = _bits((1, 3, N, d), dtype, seed=N + 1000)
    full_check(q, k, v, dtype, causal, 1 / np.sqrt(d), cfg=RUNNING,
               tag=f"running mode {dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("mode", [1, 2])
def test_peaky_long_rows_both_modes(mode):
    """Std-3 Q and K at d=128 over 1000 keys (the long workload's value
    distribution): logits with std ~9 in both exponent-reference modes."""
    B, H, N, d = 1, 8, 1000, 128
    q, k, _ = _bits((B, H, N, d), "bf16", seed=13, std=3.0)
    _, _, v = _bits((B, H, N, d), "bf16", seed=14)
    for causal in (False, True):
        full_check(q, k, v, "bf16", causal, 1 / np.sqrt(d), cfg={"mode": mode},
                   tag=f"peaky long rows mode={mode} causal={causal}")


# ---- exact properties the mathematics fixes ---------------------------------------

@pytest.mark.slow
def test_longest_sequence_closed_form():
    """The longest length the boundary admits at d = 128, N = 2^23 - 129
    (its fp32 O head plus 128 rows just fits 32-bit offsets; the last
    128-row block is ragged by one row), causal, one head.  K = 0, so every
    visible key weighs the same, and V[j, c] = ((7 j + 13 c) mod 256 - 128) / 64
    (exact in bf16).  Then O[i] is the mean of V[0..i], in closed form from
    the 256-key period of V (7 is odd, so a period holds every residue once
    and sums to -2 in every column), and LSE[i] = ln(i + 1).  Checked on rows
    at the start, at period edges and at the end, where the O store offsets
    come within 2^16 of 2^32; no row may be left unwritten."""
    import torch

    from tiled_tensor_core_amd import attn

    N, d = (1 << 23) - 129, 128
    dev = "cuda"
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros_like(q)
    j = torch.arange(N, device=dev, dtype=torch.int32)[:, None]
    c = torch.arange(d, device=dev, dtype=torch.int32)[None, :]
    v = ((((7 * j + 13 * c) % 256) - 128).to(torch.float32) / 64).to(torch.bfloat16).view(1, 1, N, d)
    del j, c
    o = torch.full((1, 1, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((1, 1, N), float("nan"), dtype=torch.float32, device=dev)
    print(f"[case] longest sequence N={N} d={d} causal", flush=True)
    attn.attn_fwd(q, k, v, o, lse, 1, 1, N, d, 1, d ** -0.5)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()) and not bool(torch.isnan(lse).any()), "a row was left unwritten"
    rows = np.array([0, 1, 2, 255, 256, 257, 4095, 1000003, N // 2, N - 257, N - 129, N - 128, N - 2, N - 1])
    rows = np.unique(np.concatenate([rows, np.random.default_rng(9).integers(0, N, 20)]))
    cc = np.arange(d)
    got_o = o[0, 0, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    got_l = lse[0, 0, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    for idx, i in enumerate(rows):
        n = int(i) + 1
        per, rem = divmod(n, 256)
        part = (((7 * np.arange(rem)[:, None] + 13 * cc[None, :]) % 256) - 128).sum(axis=0) / 64.0
        ref = (per * -2.0 + part) / n
        err_o = float(np.max(np.abs(got_o[idx] - ref)))
        err_l = abs(got_l[idx] - np.log(n))
        assert err_o <= 1e-3 and err_l <= 1e-4, f"row {i}: O error {err_o:.3e}, LSE error {err_l:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_first_causal_row_is_v0(dtype, d):
    """Causal row 0 sees key 0 only: its one P rounds to exactly 1, so O_0 is
    V_0 bit for bit in fp32, and LSE_0 is the one scaled score."""
    B, H, N = 2, 2, 200
    q, k, v = _bits((B, H, N, d), dtype, seed=21)
    o, lse = run_hip(q, k, v, dtype, True, 1 / np.sqrt(d))
    v0 = synth.bits_to_f32(v[:, :, 0], dtype)
    assert np.array_equal(o[:, :, 0].cpu().numpy(), v0)
    s00 = np.einsum("bhd,bhd->bh", synth.bits_to_f64(q[:, :, 0], dtype),
                    synth.bits_to_f64(k[:, :, 0], dtype)) / np.sqrt(d)
    np.testing.assert_allclose(lse[:, :, 0].cpu().numpy(), s00, rtol=0, atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_constant_v(dtype):
    """V_j = c for every key: O is a weighted mean of V whose weights (the
    rounded P over their sum) add up to 1, so every row is c up to fp32
    rounding of the sums."""
    B, H, N, d = 1, 2, 333, 64
    q, k, _ = _bits((B, H, N, d), dtype, seed=22)
    c = synth.round_bits(np.random.default_rng(0).standard_normal((B, H, 1, d)).astype(np.float32), dtype)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    for causal in (False, True):
        o, _ = run_hip(q, k, v, dtype, causal, 0.125)
        np.testing.assert_allclose(o.cpu().numpy(), np.broadcast_to(synth.bits_to_f32(c, dtype), o.shape),
                                   rtol=2e-6, atol=1e-7)


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


# ---- non-finite inputs -------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_inputs_follow_the_definition(dtype, d, causal):
    """A NaN in one key row reaches every query row that sees that key (all
    rows; causal: the rows at and after it) and no other; a NaN in one query
    row reaches that row only.  The NaN rows of O and LSE are exactly the
    oracle's (softmax of a row holding NaN is NaN), and the other rows meet
    the usual tolerances, although the item holding them is computed again."""
    B, H, N = 1, 2, 300
    q, k, v = _bits((B, H, N, d), dtype, seed=d + int(causal))
    nan_bits = np.uint16(0x7FC0 if dtype == "bf16" else 0x7E00)
    k[0, 0, 137, :] = nan_bits
    q[0, 1, 200, 5] = nan_bits
    o, lse = run_hip(q, k, v, dtype, causal, 1 / np.sqrt(d))
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    o_ref, lse_ref = attention_ref(synth.bits_to_f64(q, dtype), synth.bits_to_f64(k, dtype),
                                   synth.bits_to_f64(v, dtype), causal, 1 / np.sqrt(d))
    nan_rows = np.isnan(lse_ref)
    assert nan_rows.any() and not nan_rows.all()
    assert np.array_equal(np.isnan(lse), nan_rows), "LSE NaN rows differ from the oracle's"
    assert np.array_equal(np.isnan(o).any(axis=-1), nan_rows), "O NaN rows differ from the oracle's"
    assert np.array_equal(np.isnan(o).all(axis=-1), nan_rows), "a NaN row of O is only partly NaN"
    fin = ~nan_rows
    assert_close(o[fin][None], lse[fin][None], o_ref[fin][None], lse_ref[fin][None],
                 tag=f"finite rows {dtype} d={d} causal={causal}")


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


def test_concurrent_streams():
    """Calls in flight on two streams at once (different shapes, dtypes and
    masks) give what each gives alone: the fused path keeps no state between
    calls and shares no memory beyond its arguments."""
    import torch

    from tiled_tensor_core_amd import attn

    cases = [((2, 8, 900, 128), "bf16", True, 71), ((3, 5, 700, 64), "fp16", False, 72)]
    ins, alone = [], []
    for shape, dtype, causal, seed in cases:
        bits = _bits(shape, dtype, seed)
        ins.append(tuple(synth.to_torch(x, dtype, "cuda") for x in bits))
        alone.append(run_hip(*bits, dtype, causal, 1 / np.sqrt(shape[3])))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (shape, dtype, causal, _), (q, k, v) in zip(cases, ins):
        B, H, N, d = shape
        outs.append((torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda"),
                     torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    for rep in range(4):   # both streams launched back to back, several times
        for (shape, dtype, causal, _), (q, k, v), (o, lse), s in zip(cases, ins, outs, streams):
            B, H, N, d = shape
            attn.attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), 1 / np.sqrt(d), s)
    torch.cuda.synchronize()
    for (o, lse), (o1, lse1) in zip(outs, alone):
        assert torch.equal(o.view(torch.int32), o1.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))


def test_fp16_entry_rejects_nothing_valid():
    q, k, v = _bits((1, 2, 96, 128), "fp16", seed=61)
    o, lse = run_hip(q, k, v, "fp16", True, 0.1, entry="attn_fwd_fp16")
    o_ref, l_ref = attention_ref(synth.bits_to_f64(q, "fp16"), synth.bits_to_f64(k, "fp16"),
                                 synth.bits_to_f64(v, "fp16"), True, 0.1)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, tag="fp16 entry")
