"""CPU pins of the row-softmax oracle (oracle/softmax.py).

The oracle is checked against what the mathematics fixes: closed forms (two
columns give the logistic function, a constant row gives 1/n, a dominant
entry gives a one-hot row), invariants (rows sum to 1, adding a constant to
a row changes nothing, permuting columns permutes the output), an
independent scalar evaluation with math.fsum, and scipy's softmax as a
library special case.  A mutation test plants plausible mistakes in the
oracle's source and checks that a pin catches each one.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle.softmax as osm
from oracle.softmax import softmax_rows_ref


def _rand(rows, cols, seed, scale=3.0):
    return np.random.default_rng(seed).standard_normal((rows, cols)) * scale


def pin_rows_sum_to_one(fn):
    y = fn(_rand(7, 33, 1))
    return np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-14 and np.all(y >= 0)


def pin_shift_invariance(fn):
    x = _rand(5, 17, 2)
    shift = np.arange(5)[:, None] * 7.25 - 11.0
    return np.max(np.abs(fn(x + shift) - fn(x))) <= 1e-14


def pin_two_columns_logistic(fn):
    x = _rand(9, 2, 3)
    want = 1.0 / (1.0 + np.exp(x[:, 1] - x[:, 0]))
    y = fn(x)
    return np.max(np.abs(y[:, 0] - want)) <= 1e-15 and np.max(np.abs(y[:, 1] - (1 - want))) <= 1e-15


def pin_constant_row_uniform(fn):
    x = np.full((3, 11), 2.5)
    x[1] = -4.0
    return np.max(np.abs(fn(x) - 1.0 / 11)) <= 1e-16


def pin_dominant_entry_one_hot(fn):
    x = np.zeros((4, 10))
    for i in range(4):
        x[i, 3 * i % 10] = 800.0
    y = fn(x)
    want = np.zeros_like(x)
    for i in range(4):
        want[i, 3 * i % 10] = 1.0
    return np.array_equal(y, want)   # exp(-800) underflows to exactly 0 in fp64


def pin_minus_inf_weight_zero(fn):
    x = _rand(3, 8, 4)
    x[:, [1, 5]] = -np.inf
    y = fn(x)
    keep = [0, 2, 3, 4, 6, 7]
    return (np.all(y[:, [1, 5]] == 0.0)
            and np.max(np.abs(y[:, keep] - fn(x[:, keep]))) <= 1e-15)


def pin_column_permutation(fn):
    x = _rand(6, 13, 5)
    perm = np.random.default_rng(6).permutation(13)
    return np.max(np.abs(fn(x[:, perm]) - fn(x)[:, perm])) <= 1e-16


def pin_scalar_fsum(fn):
    """Independent scalar evaluation (math.exp, math.fsum) on tiny rows."""
    x = _rand(4, 9, 7, scale=5.0)
    y = fn(x)
    for i in range(x.shape[0]):
        m = max(x[i])
        e = [math.exp(v - m) for v in x[i]]
        s = math.fsum(e)
        for j in range(x.shape[1]):
            if abs(y[i, j] - e[j] / s) > 1e-15:
                return False
    return True


def pin_scipy(fn):
    special = pytest.importorskip("scipy.special")
    x = _rand(8, 65, 8)
    return np.max(np.abs(fn(x) - special.softmax(x, axis=1))) <= 1e-15


ALL_PINS = [
    ("rows_sum_to_one", pin_rows_sum_to_one),
    ("shift_invariance", pin_shift_invariance),
    ("two_columns_logistic", pin_two_columns_logistic),
    ("constant_row_uniform", pin_constant_row_uniform),
    ("dominant_entry_one_hot", pin_dominant_entry_one_hot),
    ("minus_inf_weight_zero", pin_minus_inf_weight_zero),
    ("column_permutation", pin_column_permutation),
    ("scalar_fsum", pin_scalar_fsum),
    ("scipy", pin_scipy),
]


@pytest.mark.parametrize("name", [n for n, _ in ALL_PINS])
def test_pin(name):
    assert dict(ALL_PINS)[name](softmax_rows_ref)


def test_all_minus_inf_row_is_nan():
    x = np.full((2, 5), -np.inf)
    x[1, 2] = 0.0
    y = softmax_rows_ref(x)
    assert np.all(np.isnan(y[0]))
    assert np.array_equal(y[1], [0, 0, 1, 0, 0])


def test_shapes():
    assert softmax_rows_ref(np.zeros((3, 0))).shape == (3, 0)
    assert softmax_rows_ref(np.zeros((0, 4))).shape == (0, 4)
    with pytest.raises(ValueError):
        softmax_rows_ref(np.zeros(5))


MUTATIONS = [
    ("max from the wrong axis", "m = x.max(axis=1)", "m = x.max(axis=0)[: x.shape[0]] if x.shape[0] <= x.shape[1] else x.max(axis=1)"),
    ("sum over the wrong axis", "s = e.sum(axis=1)", "s = e.sum(axis=0)[: e.shape[0]] if e.shape[0] <= e.shape[1] else e.sum(axis=1)"),
    ("normalisation dropped", "y = e / s[:, None]", "y = e"),
    ("exponent sign flipped", "e = np.exp(x - m[:, None])", "e = np.exp(m[:, None] - x)"),
    ("global maximum", "m = x.max(axis=1)", "m = np.full(x.shape[0], x.max())"),
    ("base-2 exponent", "e = np.exp(x - m[:, None])", "e = np.exp2(x - m[:, None])"),
    ("sum including the max twice", "s = e.sum(axis=1)", "s = e.sum(axis=1) + 1.0"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = inspect.getsource(osm)
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("softmax_mutant")
    exec(compile(src.replace(old, new), "softmax_mutant", "exec"), mod.__dict__)
    failed = []
    for pname, pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                ok = pin(mod.softmax_rows_ref)
        except Exception:
            ok = False
        if not ok:
            failed.append(pname)
    assert failed, f"planted mistake '{name}' passed every pin"
