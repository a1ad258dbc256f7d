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


def test_gated_rmsnorm_worked_example():
    """[3, 4] with no gate, unit weight and eps 0: the mean square is 12.5, so
    the output is [3, 4] / sqrt(12.5), worked by hand."""
    y = np.array([[[3.0, 4.0]]])          # [token, head, headdim]
    out = edges.gated_rmsnorm(y, None, np.ones(2), 0.0, 1)
    assert np.allclose(out, [[[0.848528137423857, 1.131370849898476]]], rtol=1e-14)
    # eps enters under the root: [3, 4] / sqrt(12.5 + 0.5) = [3, 4] / sqrt(13)
    out = edges.gated_rmsnorm(y, None, np.ones(2), 0.5, 1)
    assert np.allclose(out, [[[3 / np.sqrt(13.0), 4 / np.sqrt(13.0)]]], rtol=1e-14)


def test_gated_rmsnorm_unit_rms_and_weight():
    """With unit weight and eps 0 every group of the output has RMS exactly 1;
    the weight then scales each channel on its own."""
    rng = np.random.default_rng(5)
    y = rng.standard_normal((3, 7, 6, 4))  # [batch, token, head, headdim]
    z = rng.standard_normal((3, 7, 6, 4))
    out = edges.gated_rmsnorm(y, z, np.ones(24), 0.0, 3)
    g = out.reshape(3, 7, 3, 8)
    assert np.allclose(np.sqrt(np.mean(g * g, axis=-1)), 1.0, rtol=1e-13)
    w = rng.standard_normal(24)
    outw = edges.gated_rmsnorm(y, z, w, 0.0, 3)
    assert np.allclose(outw, out * w.reshape(6, 4), rtol=1e-13)


def test_gated_rmsnorm_groups_are_independent_and_scale_free():
    """Changing the heads of one group leaves the other groups' outputs alone;
    with eps 0 a positive scale of y (per group) cancels."""
    rng = np.random.default_rng(6)
    y = rng.standard_normal((5, 4, 8))      # [token, head, headdim]
    w = rng.standard_normal(32)
    out = edges.gated_rmsnorm(y, None, w, 0.0, 2)
    y2 = y.copy()
    y2[:, 2:] *= 7.5                        # group 1 (heads 2, 3) scaled
    out2 = edges.gated_rmsnorm(y2, None, w, 0.0, 2)
    assert np.array_equal(out2[:, :2], out[:, :2])
    assert np.allclose(out2[:, 2:], out[:, 2:], rtol=1e-13)
    y3 = y.copy()
    y3[:, 2:] = rng.standard_normal((5, 2, 8))
    assert np.array_equal(edges.gated_rmsnorm(y3, None, w, 0.0, 2)[:, :2], out[:, :2])


def test_gated_rmsnorm_gates_before_normalising():
    """The gate is applied before the norm: a gate that is constant over a
    group's channels (z equal everywhere) cancels in the norm (eps 0) up to
    its sign, which a gate applied after the norm would not do."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal((4, 2, 8))
    w = np.ones(16)
    z = np.full_like(y, 1.3)                # silu(1.3) > 0, the same everywhere
    assert np.allclose(edges.gated_rmsnorm(y, z, w, 0.0, 1),
                       edges.gated_rmsnorm(y, None, w, 0.0, 1), rtol=1e-13)
    # with eps > 0 the gate's size matters (a gate after the norm would scale
    # the output by exactly silu(1.3))
    a = edges.gated_rmsnorm(y, z, w, 1.0, 1)
    b = edges.gated_rmsnorm(y, None, w, 1.0, 1) * edges.silu(1.3)
    assert not np.allclose(a, b, rtol=1e-6)
