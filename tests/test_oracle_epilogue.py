"""Pins of the fused-epilogue references (no GPU).

The decode epilogues the pages fuse into the matrix kernels (aot-llm README,
Metal backend notes: biases in the epilogue of the q / k / v kernels, the
residual add fused into wo and down, one fused gate / up / SwiGLU product),
written as plain definitions in the oracle, are checked here against closed
forms of the logistic function, hand-worked values, a brute-force check of
the Lipschitz constant behind the SwiGLU bound, and planted mistakes.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import reference as ref

LN3 = math.log(3.0)


def swiglu_pins_hold(fn) -> bool:
    """Hand values: silu(0) = 0; the logistic of ln 3 is 3/4, of -ln 3 is 1/4,
    so silu(ln 3) = 0.75 ln 3, silu(-ln 3) = -0.25 ln 3; h(ln 3, 4) = 3 ln 3;
    a large negative gate gives 0, a large positive one passes g * u."""
    try:
        got = np.asarray(fn(np.array([0.0, LN3, -LN3, LN3, -80.0, 40.0]),
                            np.array([1.0, 1.0, 1.0, 4.0, 5.0, 0.5])), dtype=np.float64)
    except Exception:
        return False
    want = np.array([0.0, 0.75 * LN3, -0.25 * LN3, 3.0 * LN3, 0.0, 20.0])
    return bool(np.allclose(got, want, rtol=1e-14, atol=1e-30))


def test_swiglu_hand_values():
    assert swiglu_pins_hold(oracle.swiglu_ref)


def test_silu_odd_part_identity():
    # logistic(z) + logistic(-z) = 1  =>  silu(z) - silu(-z) = z for every z
    z = np.linspace(-30, 30, 1201)
    assert np.allclose(oracle.silu_ref(z) - oracle.silu_ref(-z), z, rtol=0, atol=1e-12)


def test_silu_lipschitz_constant_covers_the_derivative():
    # brute force over a fine grid (the derivative tends to 1 and 0 at the ends)
    z = np.linspace(-40, 40, 800001)
    s = 1.0 / (1.0 + np.exp(-z))
    d = s * (1.0 + z * (1.0 - s))
    assert np.max(np.abs(d)) <= ref.SILU_LIP
    assert np.max(np.abs(d)) > ref.SILU_LIP - 0.01  # and is not loose by much
    # the bound holds for perturbed inputs: random g, u and errors inside dg, du
    g = np.random.default_rng(3)
    gs, us = g.normal(0, 4, 20000), g.normal(0, 4, 20000)
    dg, du = np.abs(g.normal(0, 0.3, 20000)), np.abs(g.normal(0, 0.3, 20000))
    eg, eu = g.uniform(-1, 1, 20000) * dg, g.uniform(-1, 1, 20000) * du
    err = np.abs(oracle.swiglu_ref(gs + eg, us + eu) - oracle.swiglu_ref(gs, us))
    assert np.all(err <= oracle.swiglu_bound(gs, us, dg, du))


def test_epilogue_hand_values():
    y = oracle.epilogue_ref(np.array([[1.0, 2.0], [3.0, 4.0]]), bias=np.array([10.0, 20.0]),
                            residual=np.array([[100.0, 200.0], [300.0, 400.0]]))
    assert np.array_equal(y, [[111.0, 222.0], [313.0, 424.0]])
    assert np.array_equal(oracle.epilogue_ref(np.array([[1.0, 2.0]])), [[1.0, 2.0]])
    b = oracle.epilogue_bound(np.array([[0.5, 0.5]]), np.array([[1.0, 2.0]]), bias=np.array([2.0, -2.0]),
                              residual=np.array([[8.0, 0.0]]))
    assert np.array_equal(b, [[0.5 + 2.0 ** -23 * 11 + 2.0 ** -24 * 2, 0.5 + 2.0 ** -23 * 0 + 2.0 ** -24 * 2]])


def test_swiglu_mutations_are_caught():
    mutants = {
        "logistic sign flipped": lambda g, u: g / (1 + np.exp(g)) * u,
        "gate and up swapped": lambda g, u: oracle.silu_ref(u) * g,
        "logistic instead of silu": lambda g, u: u / (1 + np.exp(-g)),
        "silu of the product": lambda g, u: oracle.silu_ref(g * u),
    }
    caught = {k: not swiglu_pins_hold(f) for k, f in mutants.items()}
    assert all(caught.values()), caught


def test_epilogue_mutations_are_caught():
    yv, bias, res = np.array([[1.0, 2.0], [3.0, 4.0]]), np.array([10.0, 20.0]), np.array([[100.0, 200.0], [300.0, 400.0]])
    want = [[111.0, 222.0], [313.0, 424.0]]
    mutants = {
        "bias per vector, not per row": lambda: res + (yv + bias[:, None]),
        "residual dropped": lambda: yv + bias,
        "bias dropped": lambda: res + yv,
    }
    for name, f in mutants.items():
        assert not np.array_equal(f(), want), name
