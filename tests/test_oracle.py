"""CPU tests of the fp64 oracle against what the mathematics fixes.

The oracle (oracle/attention.py) is checked here against closed forms,
invariants, hand-derived fractions, a 50-digit evaluation and PyTorch's CPU
SDPA, and its online (tile-by-tile) recurrence against its one-shot
definition.  A mutation test plants plausible mistakes in the oracle's own
source and checks that at least one pin catches each of them.
"""

import functools
import inspect
import types

import numpy as np
import pytest

import oracle.attention as oa
from oracle import attention_online, attention_probs, attention_ref, attention_rows
from oracle_pins import ALL_PINS, PROBS_PINS, run_all, run_probs_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _online(tile):
    return lambda q, k, v, c, s: attention_online(q, k, v, c, s, tile=tile)


IMPLS = {
    "ref": attention_ref,
    "ref_chunk3": functools.partial(attention_ref, row_chunk=3),
    "online_t1": _online(1),
    "online_t4": _online(4),
    "online_t64": _online(64),
}


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("pin", [name for name, _ in ALL_PINS])
def test_pin(impl, pin):
    fn = dict(ALL_PINS)[pin]
    fn(IMPLS[impl])


@pytest.mark.parametrize("pin", [name for name, _ in PROBS_PINS])
def test_probs_pin(pin):
    dict(PROBS_PINS)[pin](attention_probs)


PROBS_MUTATIONS = [
    ("scale dropped", "s = scale * (q[b, h] @ k[b, h].T)", "s = (q[b, h] @ k[b, h].T)"),
    ("scale applied twice", "s = scale * (q[b, h] @ k[b, h].T)", "s = scale * scale * (q[b, h] @ k[b, h].T)"),
    ("q and k swapped", "s = scale * (q[b, h] @ k[b, h].T)", "s = scale * (k[b, h] @ q[b, h].T)"),
    ("mask keeps the future", "np.triu(np.ones((N, N), dtype=bool), 1)", "np.tril(np.ones((N, N), dtype=bool), -1)"),
    ("mask hides the diagonal", "np.triu(np.ones((N, N), dtype=bool), 1)", "np.triu(np.ones((N, N), dtype=bool), 0)"),
    ("normalised over the wrong axis", "p[b, h] = e / e.sum(axis=1, keepdims=True)",
     "p[b, h] = e / e.sum(axis=0, keepdims=True)"),
    ("transposed", "p[b, h] = e / e.sum(axis=1, keepdims=True)", "p[b, h] = (e / e.sum(axis=1, keepdims=True)).T"),
    ("base-2 exponent", "e = np.exp(s - m)", "e = np.exp2(s - m)"),
]


@pytest.mark.parametrize("name,old,new", PROBS_MUTATIONS, ids=[m[0] for m in PROBS_MUTATIONS])
def test_planted_mistake_in_probs_is_caught(name, old, new):
    mod = _mutant(old, new)
    assert run_probs_pins(mod.attention_probs), f"planted mistake '{name}' passed every probability pin"


@pytest.mark.parametrize("N", [1, 2, 3, 5, 17, 64])
@pytest.mark.parametrize("tile", [1, 2, 3, 4, 7, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_one_shot(N, tile, causal):
    """The tile-by-tile recurrence (running max, normaliser, rescale) reaches
    the one-shot softmax result to 1e-12, for any tile size and a ragged
    last tile."""
    rng = np.random.default_rng(N * 100 + tile)
    # std-3 inputs make peaky rows so the running max changes often
    q = rng.standard_normal((2, 2, N, 8)) * 3
    k = rng.standard_normal((2, 2, N, 8)) * 3
    v = rng.standard_normal((2, 2, N, 8))
    o1, l1 = attention_ref(q, k, v, causal, 1 / np.sqrt(8))
    o2, l2 = attention_online(q, k, v, causal, 1 / np.sqrt(8), tile=tile)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_rows_match_full():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 3, 40, 8)) for _ in range(3))
    for causal in (False, True):
        o, l = attention_ref(q, k, v, causal, 0.3)
        rows = np.array([0, 7, 39, 13])
        ro, rl = attention_rows(q, k, v, causal, 0.3, 1, 2, rows)
        assert np.array_equal(ro, o[1, 2, rows]) and np.array_equal(rl, l[1, 2, rows])


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        attention_ref(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 5, 2)), np.zeros((1, 1, 4, 2)), False, 1.0)
    with pytest.raises(ValueError):
        attention_online(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)), False, 1.0, 0)


# --- planted mistakes ------------------------------------------------------

MUTATIONS = [
    ("mask direction flipped", "key_idx > rows[:, None]", "key_idx < rows[:, None]"),
    ("mask hides the diagonal", "key_idx > rows[:, None]", "key_idx >= rows[:, None]"),
    ("mask off by one", "key_idx > rows[:, None]", "key_idx > rows[:, None] + 1"),
    ("q and k swapped", "qh[rows] @ kh.T", "kh[rows] @ qh.T"),
    ("scale dropped", "s = scale * (qh[rows] @ kh.T)", "s = (qh[rows] @ kh.T)"),
    ("scale applied twice", "s = scale * (qh[rows] @ kh.T)", "s = scale * scale * (qh[rows] @ kh.T)"),
    ("no max subtraction", "e = np.exp(s - m[:, None])", "e = np.exp(s); m = 0 * m"),
    ("max from the wrong axis", "m = s.max(axis=1)", "m = s.max(axis=1).max() + 0 * s.max(axis=1)"),
    ("normalisation dropped", "p = e / l[:, None]", "p = e"),
    ("probabilities transposed", "o = p @ vh", "o = (p.T if p.shape[0] == p.shape[1] else p) @ vh"),
    ("lse in base 2", "lse = m + np.log(l)", "lse = m + np.log2(l)"),
    ("lse without the max", "lse = m + np.log(l)", "lse = np.log(l)"),
    ("value rows shifted", "o = p @ vh", "o = p @ np.roll(vh, 1, axis=0)"),
    ("online: rescale sign", "np.exp(np.where(live, m - m_new, 0.0))", "np.exp(np.where(live, m_new - m, 0.0))"),
    ("online: l not rescaled", "l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    ("online: acc not rescaled", "acc = alpha[:, None] * acc + p @ v[b, h, cols]", "acc = acc + p @ v[b, h, cols]"),
    ("online: stale max", "p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)",
     "p = np.where(live[:, None], np.exp(s - np.where(np.isfinite(m), m, m_new)[:, None]), 0.0)"),
    ("online: causal mask flipped", "cols[None, :] > rows[:, None]", "cols[None, :] < rows[:, None]"),
    ("online: last tile dropped", "for c0 in range(0, N, tile):", "for c0 in range(0, max(N - tile, 1), tile):"),
]


def _mutant(old, new):
    src = inspect.getsource(oa)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    failed = run_all(mod.attention_ref)
    for tile in (1, 3, 16):
        failed += run_all(lambda q, k, v, c, s, t=tile: mod.attention_online(q, k, v, c, s, tile=t))
        # the recurrence must also reach the one-shot result of the unmutated oracle
        rng = np.random.default_rng(tile)
        q, k, v = (rng.standard_normal((1, 2, 19, 4)) * 2 for _ in range(3))
        for causal in (False, True):
            with np.errstate(all="ignore"):
                o1, l1 = attention_ref(q, k, v, causal, 0.5)
                o2, l2 = mod.attention_online(q, k, v, causal, 0.5, tile=tile)
            if not (np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12):
                failed.append(f"online_vs_ref_t{tile}")
    assert failed, f"planted mistake '{name}' passed every pin"
