"""CPU pins of the GEMM + bias + GELU oracle (oracle/gemm.py).

GELU is pinned by the mathematics of the standard normal distribution:
GELU(z) = z Phi(z), so GELU(0) = 0, GELU(z) - GELU(-z) = z (since Phi(z) +
Phi(-z) = 1), the slope at 0 is 1/2, and tabulated values of Phi (from -12
to 3) fix GELU at those points to a relative 1e-13 -- far in the negative
tail too, where 1 + erf(z / sqrt(2)) cancels; the tanh approximation
differs at 1e-4 and is rejected.  The product is pinned by a
brute-force triple loop on tiny non-square shapes (a transposed operand
changes the shape or the values), by the identity matrix, by a zero input
(only the bias remains) and by linearity in the bias.  A mutation test
plants plausible mistakes and checks that a pin catches each one.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle.gemm as og
from oracle.gemm import EPI_BIAS, EPI_BIAS_GELU, EPI_NONE, gelu_ref, gemm_ref

# standard normal distribution function, tabulated values
PHI = {1.0: 0.8413447460685429, -1.0: 0.15865525393145707, 1.96: 0.9750021048517795,
       3.0: 0.9986501019683699, 0.5: 0.6914624612740131, -2.0: 0.022750131948179195,
       -6.0: 9.865876450376946e-10, -12.0: 1.7764821120776e-33}


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_gelu_table(mod):
    z = np.array(list(PHI))
    want = z * np.array(list(PHI.values()))
    return np.max(np.abs(mod.gelu_ref(z) - want) / np.abs(want)) <= 1e-13


def pin_gelu_odd_part(mod):
    z = _rand(64, 1) * 4
    return np.max(np.abs(mod.gelu_ref(z) - mod.gelu_ref(-z) - z)) <= 1e-14


def pin_gelu_zero_and_slope(mod):
    h = 1e-6
    slope = (mod.gelu_ref(np.array([h]))[0] - mod.gelu_ref(np.array([-h]))[0]) / (2 * h)
    return mod.gelu_ref(np.array([0.0]))[0] == 0.0 and abs(slope - 0.5) <= 1e-9


def pin_gelu_tails(mod):
    g = mod.gelu_ref(np.array([12.0, 40.0, -40.0]))
    # Phi(-12) ~ 1.8e-33: GELU(12) = 12 to fp64 precision; GELU(-40) underflows to -0
    return g[0] == 12.0 and g[1] == 40.0 and g[2] == 0.0


def pin_brute_force(mod):
    a, w, b = _rand((3, 5), 2), _rand((4, 5), 3), _rand(4, 4)
    want = np.zeros((3, 4))
    for i in range(3):
        for j in range(4):
            s = math.fsum(a[i, k] * w[j, k] for k in range(5)) + b[j]
            want[i, j] = s * 0.5 * (1.0 + math.erf(s / math.sqrt(2.0)))
    got = mod.gemm_ref(a, w, b, mod.EPI_BIAS_GELU)
    return got.shape == (3, 4) and np.max(np.abs(got - want)) <= 1e-14


def pin_no_epilogue(mod):
    a, w = _rand((2, 7), 5), _rand((3, 7), 6)
    want = np.array([[math.fsum(a[i, k] * w[j, k] for k in range(7)) for j in range(3)] for i in range(2)])
    return np.max(np.abs(mod.gemm_ref(a, w, None, mod.EPI_NONE) - want)) <= 1e-14


def pin_identity(mod):
    a = _rand((6, 6), 7)
    b = _rand(6, 8)
    return (np.max(np.abs(mod.gemm_ref(a, np.eye(6), b, mod.EPI_BIAS) - (a + b[None, :]))) <= 1e-15)


def pin_zero_input_leaves_bias(mod):
    b = np.array([-2.0, 0.0, 1.0, 3.0])
    got = mod.gemm_ref(np.zeros((2, 3)), _rand((4, 3), 9), b, mod.EPI_BIAS_GELU)
    want = b * np.array([PHI[-2.0], 0.0, PHI[1.0], PHI[3.0]])
    return np.max(np.abs(got - want[None, :])) <= 1e-15


def pin_bias_linearity(mod):
    a, w = _rand((3, 4), 10), _rand((5, 4), 11)
    b1, b2 = _rand(5, 12), _rand(5, 13)
    z1 = mod.gemm_ref(a, w, b1, mod.EPI_BIAS)
    z2 = mod.gemm_ref(a, w, b2, mod.EPI_BIAS)
    return np.max(np.abs((z1 - z2) - (b1 - b2)[None, :])) <= 1e-14


ALL_PINS = [
    ("gelu_table", pin_gelu_table),
    ("gelu_odd_part", pin_gelu_odd_part),
    ("gelu_zero_and_slope", pin_gelu_zero_and_slope),
    ("gelu_tails", pin_gelu_tails),
    ("brute_force", pin_brute_force),
    ("no_epilogue", pin_no_epilogue),
    ("identity", pin_identity),
    ("zero_input_leaves_bias", pin_zero_input_leaves_bias),
    ("bias_linearity", pin_bias_linearity),
]


@pytest.mark.parametrize("name", [n for n, _ in ALL_PINS])
def test_pin(name):
    assert dict(ALL_PINS)[name](og)


def test_tanh_approximation_is_not_the_reading():
    z = np.array([1.0])
    tanh_form = 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert abs(gelu_ref(z)[0] - tanh_form[0]) > 1e-4


def test_shapes_and_errors():
    assert gemm_ref(np.zeros((0, 4)), np.zeros((3, 4)), np.zeros(3)).shape == (0, 3)
    assert gemm_ref(np.zeros((2, 0)), np.zeros((3, 0)), np.ones(3), EPI_BIAS).tolist() == [[1, 1, 1]] * 2
    with pytest.raises(ValueError):
        gemm_ref(np.zeros((2, 3)), np.zeros((3, 4)), np.zeros(3))
    with pytest.raises(ValueError):
        gemm_ref(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros(3))
    with pytest.raises(ValueError):
        gemm_ref(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros(4), epilogue=5)


MUTATIONS = [
    ("W not transposed", "z = a @ w.T", "z = a @ w"),
    ("bias on the rows", "z = z + b[None, :]", "z = z + b[:z.shape[0], None] if z.shape[0] <= b.shape[0] else z + b[None, :]"),
    ("erfc argument not scaled", "erfc(-z / np.sqrt(2.0))", "erfc(-z)"),
    ("half dropped", "return z * (0.5 * erfc", "return z * (1.0 * erfc"),
    ("tanh approximation", "return z * (0.5 * erfc(-z / np.sqrt(2.0)))",
     "return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))"),
    ("the cancelling 1 + erf form", "return z * (0.5 * erfc(-z / np.sqrt(2.0)))",
     "return 0.5 * z * (2.0 - erfc(z / np.sqrt(2.0)))"),
    ("bias after GELU", "    z = z + b[None, :]\n    if epilogue == EPI_BIAS:\n        return z\n    return gelu_ref(z)",
     "    if epilogue == EPI_BIAS:\n        return z + b[None, :]\n    return gelu_ref(z) + b[None, :]"),
    ("sign of the erfc argument flipped", "erfc(-z / np.sqrt(2.0))", "erfc(z / np.sqrt(2.0))"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = inspect.getsource(og)
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("gemm_mutant")
    exec(compile(src.replace(old, new), "gemm_mutant", "exec"), mod.__dict__)
    failed = []
    for pname, pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                ok = pin(mod)
        except Exception:
            ok = False
        if not ok:
            failed.append(pname)
    assert failed, f"planted mistake '{name}' passed every pin"
