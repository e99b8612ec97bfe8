"""Pins for the fp64 oracle: checks against facts that the mathematics of
scaled dot-product attention fixes, independent of how the oracle computes.

Each pin takes an implementation ``impl(q, k, v, causal, scale) -> (O, LSE)``
so the same checks run on the one-shot oracle, on the tile-by-tile online
recurrence, and on mutants of the oracle with planted mistakes.  A pin raises
AssertionError when the implementation disagrees with the fact.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(shape, seed, scale=1.0):
    return _rng(seed).standard_normal(shape) * scale


def _visible_counts(N, causal):
    return np.arange(1, N + 1) if causal else np.full(N, N)


def pin_constant_v(impl, N=13, d=8, causal=False):
    """V_j = c for every key: every output row is exactly c (weights sum to 1)."""
    q = _rand((2, 3, N, d), 1)
    k = _rand((2, 3, N, d), 2)
    c = _rand((2, 3, 1, d), 3)
    v = np.broadcast_to(c, (2, 3, N, d)).copy()
    o, _ = impl(q, k, v, causal, 0.37)
    err = np.max(np.abs(o - c))
    assert err <= 1e-14 * max(1.0, np.max(np.abs(c))), f"constant V: err {err}"


def pin_first_causal_row(impl, N=9, d=16):
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    q = _rand((1, 2, N, d), 4)
    k = _rand((1, 2, N, d), 5)
    v = _rand((1, 2, N, d), 6)
    scale = 0.25
    o, lse = impl(q, k, v, True, scale)
    assert np.array_equal(o[:, :, 0], v[:, :, 0]), "causal row 0 must equal V[0]"
    want = scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - want)) <= 1e-14 * max(1, np.max(np.abs(want))), \
        "causal LSE_0 must be the single scaled score"


def pin_equal_keys(impl, N=11, d=8, causal=False, logit=None):
    """K_j = k for all j: uniform weights 1/n_i over the visible keys.

    O_i = mean(V_0 .. V_{n_i-1}) and LSE_i = scale q_i . k + ln n_i, with
    n_i = N (non-causal) or i + 1 (causal).  With ``logit`` set, q and k are
    chosen so every score is about ``logit`` (tests large magnitudes)."""
    q = _rand((2, 2, N, d), 7)
    kk = _rand((2, 2, 1, d), 8)
    if logit is not None:
        # make the scores of row i ~ logit_i: q_i = logit_i * k / |k|^2
        # (+ small noise); a per-row array mixes magnitudes across rows
        kn = np.sum(kk * kk, axis=-1, keepdims=True)
        lg = np.broadcast_to(np.asarray(logit, dtype=np.float64), (N,))[None, None, :, None]
        q = lg * kk / kn + 1e-3 * q
    k = np.broadcast_to(kk, (2, 2, N, d)).copy()
    v = _rand((2, 2, N, d), 9)
    scale = 1.0 if logit is not None else 0.3
    o, lse = impl(q, k, v, causal, scale)
    n = _visible_counts(N, causal)
    want_o = np.cumsum(v, axis=2) / n[None, None, :, None] if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    want_lse = scale * np.einsum("bhnd,bhd->bhn", q, kk[:, :, 0]) + np.log(n)[None, None, :]
    assert np.max(np.abs(o - want_o)) <= 1e-12, "equal keys must give uniform weights"
    tol = 1e-12 * max(1.0, float(np.max(np.abs(want_lse))))
    assert np.max(np.abs(lse - want_lse)) <= tol, "equal keys: LSE = score + ln n"


def pin_single_key(impl, d=5):
    """N = 1: O = V and LSE = scale q . k, causal or not."""
    q, k, v = _rand((3, 2, 1, d), 10), _rand((3, 2, 1, d), 11), _rand((3, 2, 1, d), 12)
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, 0.7)
        assert np.array_equal(o, v)
        want = 0.7 * np.sum(q * k, axis=-1)
        assert np.max(np.abs(lse - want)) <= 1e-14 * max(1, np.max(np.abs(want)))


def pin_zero_scale(impl, N=10, d=4, causal=True):
    """scale = 0: all scores are 0, so O_i is the mean of the visible V rows
    and LSE_i = ln n_i."""
    q, k, v = _rand((1, 2, N, d), 13), _rand((1, 2, N, d), 14), _rand((1, 2, N, d), 15)
    o, lse = impl(q, k, v, causal, 0.0)
    n = _visible_counts(N, causal)
    want_o = np.cumsum(v, axis=2) / n[None, None, :, None] if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.max(np.abs(o - want_o)) <= 1e-13
    assert np.max(np.abs(lse - np.log(n))) <= 1e-13


def pin_key_shift(impl, N=12, d=6, causal=False):
    """Adding u to every key adds scale q_i . u to every score of row i:
    the softmax is unchanged, LSE_i shifts by exactly that amount."""
    q, k, v = _rand((1, 3, N, d), 16), _rand((1, 3, N, d), 17), _rand((1, 3, N, d), 18)
    u = _rand((1, 3, 1, d), 19)
    scale = 0.45
    o1, l1 = impl(q, k, v, causal, scale)
    o2, l2 = impl(q, k + u, v, causal, scale)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    shift = scale * np.einsum("bhnd,bhd->bhn", q, u[:, :, 0])
    assert np.max(np.abs((l2 - l1) - shift)) <= 1e-12


def pin_permutations(impl, N=9, d=4):
    """Non-causal: permuting (K, V) rows jointly changes nothing; permuting
    the Q rows permutes the output rows the same way."""
    q, k, v = _rand((1, 2, N, d), 20), _rand((1, 2, N, d), 21), _rand((1, 2, N, d), 22)
    o, lse = impl(q, k, v, False, 0.6)
    pk = _rng(23).permutation(N)
    o2, lse2 = impl(q, k[:, :, pk], v[:, :, pk], False, 0.6)
    assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13
    pq = _rng(24).permutation(N)
    o3, lse3 = impl(q[:, :, pq], k, v, False, 0.6)
    assert np.max(np.abs(o[:, :, pq] - o3)) <= 1e-13
    assert np.max(np.abs(lse[:, :, pq] - lse3)) <= 1e-13


def pin_linear_in_v(impl, N=8, d=3, causal=True):
    """O is linear in V for fixed Q, K."""
    q, k = _rand((1, 1, N, d), 25), _rand((1, 1, N, d), 26)
    v1, v2 = _rand((1, 1, N, d), 27), _rand((1, 1, N, d), 28)
    a, b = 1.7, -0.4
    o1, _ = impl(q, k, v1, causal, 0.5)
    o2, _ = impl(q, k, v2, causal, 0.5)
    o3, _ = impl(q, k, a * v1 + b * v2, causal, 0.5)
    assert np.max(np.abs(o3 - (a * o1 + b * o2))) <= 1e-13


def pin_golden(impl):
    """Hand-derived closed forms (tests/golden/closed_form_weights.json)."""
    with open(os.path.join(GOLDEN, "closed_form_weights.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w = np.array(c["w"], dtype=np.float64)
        n = len(w)
        q = np.tile(np.array([1.0, 0.0]), (n, 1))
        k = np.stack([np.log(w) + c["shift"], np.array(c["k_second"], dtype=np.float64)], axis=1)
        v = np.array(c["v"], dtype=np.float64)
        o, lse = impl(q[None, None], k[None, None], v[None, None], c["causal"], 1.0)
        want_o = np.array([[float(Fraction(x)) for x in row] for row in c["expected_o"]])
        want_lse = c["shift"] + np.log(np.array(c["expected_lse_ln_of"], dtype=np.float64))
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), c["name"]
        assert np.max(np.abs(o[0, 0] - want_o)) <= 1e-13, c["name"]
        assert np.max(np.abs(lse[0, 0] - want_lse)) <= 1e-12 * max(1, abs(c["shift"])), c["name"]


def mp_attention(q, k, v, causal, scale, digits=50):
    """50-digit evaluation of one head with mpmath (tiny shapes only)."""
    import mpmath

    mpmath.mp.dps = digits
    N, d = q.shape
    o = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(N):
        vis = range(i + 1) if causal else range(N)
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, c]) * mpmath.mpf(k[j, c])
                                             for c in range(d)) for j in vis]
        z = mpmath.fsum(mpmath.exp(x) for x in s)
        for c in range(d):
            o[i, c] = float(mpmath.fsum(mpmath.exp(x) * mpmath.mpf(v[j, c])
                                        for x, j in zip(s, vis)) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse


def pin_high_precision(impl, N=6, d=3):
    """Against a 50-digit evaluation: agreement to fp64 rounding."""
    q, k, v = _rand((1, 1, N, d), 29, 2.0), _rand((1, 1, N, d), 30, 2.0), _rand((1, 1, N, d), 31)
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, 0.8)
        wo, wl = mp_attention(q[0, 0], k[0, 0], v[0, 0], causal, 0.8)
        assert np.max(np.abs(o[0, 0] - wo)) <= 1e-13
        assert np.max(np.abs(lse[0, 0] - wl)) <= 1e-13


def pin_torch_sdpa(impl, N=33, d=16):
    """PyTorch's own scaled dot-product attention on the CPU in float64 (the
    routine the pages validate against), and logsumexp of the scaled scores."""
    import torch

    q, k, v = _rand((2, 2, N, d), 32), _rand((2, 2, N, d), 33), _rand((2, 2, N, d), 34)
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, 0.21)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        want = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.21).numpy()
        s = 0.21 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        want_lse = torch.logsumexp(s, dim=-1).numpy()
        assert np.max(np.abs(o - want)) <= 1e-12
        assert np.max(np.abs(lse - want_lse)) <= 1e-12


ALL_PINS = [
    ("constant_v", lambda f: (pin_constant_v(f, causal=False), pin_constant_v(f, causal=True))),
    ("first_causal_row", pin_first_causal_row),
    ("equal_keys", lambda f: (pin_equal_keys(f, causal=False), pin_equal_keys(f, causal=True))),
    ("equal_keys_large_logits", lambda f: (pin_equal_keys(f, causal=True, logit=900.0),
                                           pin_equal_keys(f, causal=False, logit=-900.0))),
    ("equal_keys_mixed_rows", lambda f: (
        pin_equal_keys(f, causal=True, logit=np.where(np.arange(11) % 2 == 0, 800.0, -800.0)),
        pin_equal_keys(f, causal=False, logit=np.linspace(-700.0, 700.0, 11)))),
    ("single_key", pin_single_key),
    ("zero_scale", lambda f: (pin_zero_scale(f, causal=True), pin_zero_scale(f, causal=False))),
    ("key_shift", lambda f: (pin_key_shift(f, causal=False), pin_key_shift(f, causal=True))),
    ("permutations", pin_permutations),
    ("linear_in_v", pin_linear_in_v),
    ("golden", pin_golden),
    ("high_precision", pin_high_precision),
    ("torch_sdpa", pin_torch_sdpa),
]


def run_all(impl):
    """Run every pin; return the names of the ones that fail."""
    failed = []
    for name, pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(name)
    return failed


# ---- pins of the probability matrix P (attention_probs) -------------------------
# Each takes ``probs_fn(q, k, causal, scale) -> P [B, H, N, N]``.

def probs_pin_golden(probs_fn):
    """The hand-derived cases of tests/golden/closed_form_weights.json: with
    q_i = [1, 0] and k_j = [ln w_j + shift, *] at scale 1, P_ij is the exact
    fraction w_j / (sum of w over the keys row i sees)."""
    with open(os.path.join(GOLDEN, "closed_form_weights.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w = [Fraction(x) for x in c["w"]]
        n = len(w)
        q = np.tile(np.array([1.0, 0.0]), (n, 1))
        k = np.stack([np.log(np.array(c["w"], dtype=np.float64)) + c["shift"],
                      np.array(c["k_second"], dtype=np.float64)], axis=1)
        p = probs_fn(q[None, None], k[None, None], c["causal"], 1.0)[0, 0]
        want = np.zeros((n, n))
        for i in range(n):
            vis = range(i + 1) if c["causal"] else range(n)
            tot = sum(w[j] for j in vis)
            for j in vis:
                want[i, j] = float(w[j] / tot)
        assert np.max(np.abs(p - want)) <= 1e-13, c["name"]


def probs_pin_log_ratio(probs_fn, N=7, d=5):
    """Non-causal: ln P_ij - ln P_i0 = scale q_i . (k_j - k_0) exactly in real
    arithmetic, whatever the normaliser; this fixes the scale, which operand
    is the query, and that row i of P belongs to query i."""
    q, k = _rand((1, 2, N, d), 37), _rand((1, 2, N, d), 38)
    scale = 0.6
    p = probs_fn(q, k, False, scale)
    got = np.log(p) - np.log(p[..., :1])
    want = scale * np.einsum("bhid,bhjd->bhij", q, k - k[:, :, :1])
    assert np.max(np.abs(got - want)) <= 1e-12


def probs_pin_high_precision(probs_fn, N=5, d=3):
    """Every entry of P against a 50-digit evaluation, causal and not."""
    import mpmath

    mpmath.mp.dps = 50
    q, k = _rand((1, 1, N, d), 39, 2.0), _rand((1, 1, N, d), 40, 2.0)
    for causal in (False, True):
        p = probs_fn(q, k, causal, 0.8)[0, 0]
        for i in range(N):
            vis = range(i + 1) if causal else range(N)
            s = {j: mpmath.mpf(0.8) * mpmath.fsum(mpmath.mpf(q[0, 0, i, c]) * mpmath.mpf(k[0, 0, j, c])
                                                  for c in range(d)) for j in vis}
            z = mpmath.fsum(mpmath.exp(x) for x in s.values())
            for j in range(N):
                want = float(mpmath.exp(s[j]) / z) if j in s else 0.0
                assert abs(p[i, j] - want) <= 1e-15, (causal, i, j)


def probs_pin_times_v(probs_fn, N=11, d=4):
    """P V and the row log-sum-exp reproduce the pinned one-shot oracle:
    O = P V, and for every visible key ln P_ij = scale q_i . k_j - LSE_i."""
    from oracle import attention_ref

    q, k, v = _rand((2, 2, N, d), 41), _rand((2, 2, N, d), 42), _rand((2, 2, N, d), 43)
    for causal in (False, True):
        p = probs_fn(q, k, causal, 0.45)
        o, lse = attention_ref(q, k, v, causal, 0.45)
        assert np.max(np.abs(p @ v - o)) <= 1e-13
        s = 0.45 * np.einsum("bhid,bhjd->bhij", q, k)
        vis = ~np.triu(np.ones((N, N), dtype=bool), 1) if causal else np.ones((N, N), dtype=bool)
        with np.errstate(divide="ignore"):
            lp = np.log(p)
        assert np.max(np.abs((lp - (s - lse[..., None]))[..., vis])) <= 1e-12


PROBS_PINS = [
    ("rows_sum_to_one", lambda f: softmax_rows_sum_to_one(f)),
    ("golden", probs_pin_golden),
    ("log_ratio", probs_pin_log_ratio),
    ("high_precision", probs_pin_high_precision),
    ("times_v", probs_pin_times_v),
]


def run_probs_pins(probs_fn):
    failed = []
    for name, pin in PROBS_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(probs_fn)
        except (AssertionError, ValueError, FloatingPointError, IndexError, KeyError):
            failed.append(name)
    return failed


def softmax_rows_sum_to_one(probs_fn, N=15, d=8):
    """Every row of P sums to 1 and masked entries are exactly 0."""
    q, k = _rand((2, 2, N, d), 35), _rand((2, 2, N, d), 36)
    for causal in (False, True):
        p = probs_fn(q, k, causal, 0.5)
        assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-14
        assert np.all(p >= 0)
        if causal:
            assert np.all(p[..., np.triu(np.ones((N, N), dtype=bool), 1)] == 0.0)

