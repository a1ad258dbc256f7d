"""Pins for the fp64 edge functions of the oracle (dt activation and output
gate), each against a closed form, an identity or an independent library
routine rather than against itself."""
import math

import numpy as np
import scipy.special

from oracle import edges


def test_softplus_closed_forms():
    assert abs(edges.softplus(0.0) - math.log(2.0)) < 1e-15
    # log(1 + e^v) - log(1 + e^-v) = v for every v
    v = np.linspace(-30, 30, 601)
    assert np.max(np.abs(edges.softplus(v) - edges.softplus(-v) - v)) < 1e-13
    # the two tails: v itself above, e^v below
    assert edges.softplus(60.0) == 60.0
    assert abs(edges.softplus(-40.0) / math.exp(-40.0) - 1.0) < 1e-15
    # monotone and positive
    s = edges.softplus(v)
    assert np.all(s > 0) and np.all(np.diff(s) > 0)


def test_softplus_inverts_the_bias_rule():
    """The block sets its bias to softplus^-1(dt0) so that softplus(bias) is dt0
    (repository tour, "Why You Need This"); log(expm1(dt0)) is that inverse."""
    dt0 = np.exp(np.linspace(math.log(1e-3), math.log(0.1), 50))
    bias = np.log(np.expm1(dt0))
    assert np.max(np.abs(edges.softplus(bias) / dt0 - 1.0)) < 1e-12


def test_dt_activation_order_and_broadcast():
    rng = np.random.default_rng(0)
    dt = rng.standard_normal((2, 7, 3))
    bias = np.array([-2.0, 0.5, 3.0])
    # nothing requested: the identity
    assert np.array_equal(edges.dt_activation(dt), dt)
    # bias is per head (last axis)
    assert np.array_equal(edges.dt_activation(dt, bias), dt + bias[None, None, :])
    # softplus of the biased value
    got = edges.dt_activation(dt, bias, softplus_on=True)
    assert np.max(np.abs(got - np.log1p(np.exp(dt + bias)))) < 1e-14
    # the clamp acts after the softplus: a very negative input lands on lo
    # exactly (clamping first would give softplus(lo) instead)
    lo, hi = 1e-3, 0.1
    d = edges.dt_activation(np.array([-50.0, 0.0, 50.0]), softplus_on=True, limit=(lo, hi))
    assert d[0] == lo and d[2] == hi and abs(d[1] - hi) == 0.0  # softplus(0) = ln 2 > hi
    d = edges.dt_activation(np.array([-3.0]), softplus_on=True, limit=(lo, hi))
    assert abs(d[0] - math.log1p(math.exp(-3.0))) < 1e-15  # inside the range: untouched


def test_silu_closed_forms():
    v = np.linspace(-20, 20, 401)
    assert edges.silu(0.0) == 0.0
    # silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1)
    assert np.max(np.abs(edges.silu(v) - edges.silu(-v) - v)) < 1e-13
    # against scipy's logistic function
    assert np.max(np.abs(edges.silu(v) - v * scipy.special.expit(v))) < 1e-14
    # slope 1/2 at 0
    h = 1e-6
    assert abs((edges.silu(h) - edges.silu(-h)) / (2 * h) - 0.5) < 1e-9
    # tails: v above, 0 below (no overflow warning or NaN)
    assert edges.silu(50.0) == 50.0
    assert edges.silu(-800.0) == 0.0


def test_gate_is_linear_in_y():
    rng = np.random.default_rng(1)
    y, y2, z = rng.standard_normal((3, 5, 4))
    assert np.max(np.abs(edges.gate(y + 2 * y2, z)
                         - (edges.gate(y, z) + 2 * edges.gate(y2, z)))) < 1e-14
    assert np.array_equal(edges.gate(y, np.zeros_like(z)), np.zeros_like(y))
