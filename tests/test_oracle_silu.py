"""The oracle's SiLU-gated product (silu_mul: y = silu(g) * u, silu(g) = g/(1+e^-g)),
pinned to facts that do not come from its own formula: an independent form through
tanh, the odd-part identity, limits, the slope at zero, and the asymmetry between
the gate and the up operand."""
import math

import numpy as np
import pytest

import oracle


def test_independent_tanh_form():
    # silu(x) = x * (1 + tanh(x/2)) / 2, the logistic function through tanh; below
    # -4 that form cancels, so the tail uses x e^x / (1 + e^x) (exp of +x, not -x)
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.standard_normal(2000) * 4, np.linspace(-30, 30, 601)])
    u = rng.standard_normal(g.size)
    sig = np.where(g >= -4, (1.0 + np.tanh(g / 2.0)) / 2.0, np.exp(g) / (1.0 + np.exp(g)))
    want = g * sig * u
    got = oracle.silu_mul(g, u)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300)


def test_odd_part_identity():
    # silu(x) - silu(-x) = x exactly in the reals
    x = np.linspace(-12, 12, 481)
    one = np.ones_like(x)
    diff = oracle.silu_mul(x, one) - oracle.silu_mul(-x, one)
    assert np.allclose(diff, x, rtol=1e-14, atol=1e-14)


def test_zero_limits_and_slope():
    one = np.ones(1)
    assert oracle.silu_mul(np.zeros(1), np.array([7.5]))[0] == 0.0
    assert oracle.silu_mul(np.array([40.0]), one)[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu_mul(np.array([-40.0]), one)[0]) < 40 * math.exp(-40) * 1.0001
    h = 1e-6
    slope = (oracle.silu_mul(np.array([h]), one)[0] - oracle.silu_mul(np.array([-h]), one)[0]) / (2 * h)
    assert slope == pytest.approx(0.5, abs=1e-9)


def test_gate_and_up_not_interchangeable():
    # silu(2) * 3 = 2 * 3 / (1 + e^-2); the swapped product silu(3) * 2 differs
    got = oracle.silu_mul(np.array([2.0]), np.array([3.0]))[0]
    assert got == pytest.approx(6.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert abs(got - 6.0 / (1.0 + math.exp(-3.0))) > 0.1


def test_linear_in_up_operand():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(100)
    u = rng.standard_normal(100)
    a = oracle.silu_mul(g, u)
    b = oracle.silu_mul(g, 2.0 * u)
    assert np.array_equal(2.0 * a, b)
