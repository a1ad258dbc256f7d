"""Pins for the oracle's gradient (adjoint recurrence): every input's
gradient against central finite differences of the forward oracle (itself
pinned in test_oracle.py), along random directions, in fp64.

J(theta) = sum(dy * y) + sum(dfinal * final); for a direction V of input X,
(J(X + eps V) - J(X - eps V)) / (2 eps) = <dJ/dX, V> + O(eps^2)."""
import numpy as np
import pytest

import oracle
from mamba_ssd_chunked_scan_amd import synth

KEYS = ("x", "dt", "A", "B", "C", "D", "init")


def problem(Bt, L, H, P, N, G, seed):
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=16, dtype="f32", dt_rule="shifted",
                             init="normal", seed=seed)
    inp = {k: oracle.f64(v) for k, v in synth.scan_inputs(spec).items()}
    rng = np.random.default_rng(seed + 100)
    dy = rng.standard_normal(inp["x"].shape)
    dfinal = rng.standard_normal(inp["init"].shape)
    return inp, dy, dfinal


def J(inp, dy, dfinal):
    y, fin = oracle.scan(**inp)
    return float(np.sum(dy * y) + np.sum(dfinal * fin))


@pytest.mark.parametrize("Bt,L,H,P,N,G", [(2, 13, 4, 3, 5, 2), (1, 40, 2, 2, 4, 1)])
def test_vjp_matches_finite_differences(Bt, L, H, P, N, G):
    inp, dy, dfinal = problem(Bt, L, H, P, N, G, seed=L)
    g = oracle.scan_vjp(**inp, dy=dy, dfinal=dfinal)
    rng = np.random.default_rng(7)
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}
    for k in KEYS:
        V = rng.standard_normal(inp[k].shape)
        eps = 1e-6 * max(1.0, float(np.max(np.abs(inp[k]))))
        plus = dict(inp, **{k: inp[k] + eps * V})
        minus = dict(inp, **{k: inp[k] - eps * V})
        fd = (J(plus, dy, dfinal) - J(minus, dy, dfinal)) / (2 * eps)
        an = float(np.sum(g[names[k]] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, fd, an)


def test_vjp_without_final_term_and_without_D():
    """dfinal = None drops the final-state term; D = None gives the same dx as
    D = 0, and dD is still the gradient a D would receive."""
    inp, dy, _ = problem(1, 20, 2, 3, 4, 1, seed=3)
    g1 = oracle.scan_vjp(**inp, dy=dy, dfinal=None)
    g0 = oracle.scan_vjp(**inp, dy=dy, dfinal=np.zeros_like(inp["init"]))
    for k in g1:
        assert np.array_equal(g1[k], g0[k]), k
    noD = dict(inp, D=None)
    zD = dict(inp, D=np.zeros_like(inp["D"]))
    a, b = oracle.scan_vjp(**noD, dy=dy), oracle.scan_vjp(**zD, dy=dy)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    # dD is the sum over tokens and channels of dy * x
    assert np.allclose(a["dD"], np.einsum("blhp,blhp->h", dy, inp["x"]), rtol=1e-13)


def test_vjp_is_deterministic():
    inp, dy, dfinal = problem(3, 17, 4, 2, 4, 2, seed=9)
    a = oracle.scan_vjp(**inp, dy=dy, dfinal=dfinal, nthreads=3)
    b = oracle.scan_vjp(**inp, dy=dy, dfinal=dfinal, nthreads=1)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _edge_problem(Bt, L, H, P, N, G, seed):
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=16, dtype="f32", dt_rule="ranged",
                             init="normal", seed=seed)
    inp = {k: oracle.f64(v) for k, v in synth.scan_edge_inputs(spec).items()}
    rng = np.random.default_rng(seed + 200)
    return inp, rng.standard_normal(inp["x"].shape), rng.standard_normal(inp["init"].shape)


def _J_edges(inp, dy, dfinal, limit, gated):
    from oracle import edges
    dt = edges.dt_activation(inp["dt_raw"], inp["dt_bias"], True, limit)
    y, fin = oracle.scan(inp["x"], dt, inp["A"], inp["B"], inp["C"], inp["D"], inp["init"])
    if gated:
        y = edges.gate(y, inp["gate"])
    return float(np.sum(dy * y) + np.sum(dfinal * fin))


@pytest.mark.parametrize("limit", [None, (1e-3, 0.05)])
@pytest.mark.parametrize("gated", [True, False])
def test_vjp_edges_matches_finite_differences(limit, gated):
    """The gradient through the fused edges (bias, softplus, optional clamp,
    optional gate) against central differences of the composite forward, for
    every input it adds or changes: dt_raw, dt_bias, z, and x and B through
    the gated path.  The clamp's upper bound sits inside the range of the
    synthetic dt, so some elements are held at it (gradient 0)."""
    inp, dy, dfinal = _edge_problem(2, 11, 4, 3, 5, 2, seed=17)
    g = oracle.scan_vjp_edges(inp["x"], inp["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["init"], dy=dy, dfinal=dfinal, dt_bias=inp["dt_bias"],
                              dt_softplus=True, dt_limit=limit,
                              z=inp["gate"] if gated else None)
    if limit is not None:
        from oracle import edges
        pre = edges.softplus(inp["dt_raw"] + inp["dt_bias"])
        assert np.any(pre > limit[1]) and np.any(g["ddt"] == 0.0)
    rng = np.random.default_rng(9)
    checks = [("dt_raw", "ddt"), ("dt_bias", "ddt_bias"), ("x", "dx"), ("B", "dB")]
    if gated:
        checks.append(("gate", "dz"))
    for k, gk in checks:
        V = rng.standard_normal(inp[k].shape)
        eps = 1e-6 * max(1.0, float(np.max(np.abs(inp[k]))))
        plus = dict(inp, **{k: inp[k] + eps * V})
        minus = dict(inp, **{k: inp[k] - eps * V})
        fd = (_J_edges(plus, dy, dfinal, limit, gated)
              - _J_edges(minus, dy, dfinal, limit, gated)) / (2 * eps)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, fd, an)
    if not gated:
        assert "dz" not in g



@pytest.mark.parametrize("gated,groups", [(True, 2), (False, 1)])
def test_vjp_edges_norm_matches_finite_differences(gated, groups):
    """The gradient through the gated RMSNorm as well: dnorm_weight, z, dt_raw
    and x against central differences of the composite forward
    (edges.gated_rmsnorm after the gated scan)."""
    from oracle import edges
    inp, dy, dfinal = _edge_problem(2, 9, 4, 3, 5, 2, seed=23)
    rng = np.random.default_rng(24)
    inp["normw"] = 1.0 + 0.5 * rng.standard_normal(4 * 3)
    eps = 1e-3

    def J(q):
        dt = edges.dt_activation(q["dt_raw"], q["dt_bias"], True, None)
        y, fin = oracle.scan(q["x"], dt, q["A"], q["B"], q["C"], q["D"], q["init"])
        y = edges.gated_rmsnorm(y, q["gate"] if gated else None, q["normw"], eps, groups)
        return float(np.sum(dy * y) + np.sum(dfinal * fin))

    g = oracle.scan_vjp_edges(inp["x"], inp["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["init"], dy=dy, dfinal=dfinal, dt_bias=inp["dt_bias"],
                              dt_softplus=True, z=inp["gate"] if gated else None,
                              norm_weight=inp["normw"], norm_eps=eps, norm_groups=groups)
    checks = [("normw", "dnorm_weight"), ("dt_raw", "ddt"), ("x", "dx"), ("dt_bias", "ddt_bias")]
    if gated:
        checks.append(("gate", "dz"))
    for k, gk in checks:
        V = rng.standard_normal(inp[k].shape)
        h = 1e-6 * max(1.0, float(np.max(np.abs(inp[k]))))
        fd = (J(dict(inp, **{k: inp[k] + h * V})) - J(dict(inp, **{k: inp[k] - h * V}))) / (2 * h)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, fd, an)


def test_vjp_varlen_matches_finite_differences():
    """The ragged batch's gradient (per-sequence adjoints, an empty sequence
    passing dfinal to dinit) against central differences of the ragged
    forward oracle, for every input."""
    lengths = [5, 0, 9, 3]
    vin = {k: oracle.f64(v) if k != "cu_seqlens" else v.numpy()
           for k, v in synth.varlen_inputs(lengths, 3, 2, 4, 1, "f32", seed=71).items()}
    rng = np.random.default_rng(72)
    dy = rng.standard_normal(vin["x"].shape)
    dfinal = rng.standard_normal(vin["init"].shape)
    keys = ("x", "dt", "A", "B", "C", "D", "init")

    def J(q):
        y, fin = oracle.scan_varlen(vin["cu_seqlens"], q["x"], q["dt"], q["A"], q["B"], q["C"],
                                    q["D"], q["init"])
        return float(np.sum(dy * y) + np.sum(dfinal * fin))

    g = oracle.scan_vjp_varlen(vin["cu_seqlens"], vin["x"], vin["dt"], vin["A"], vin["B"],
                               vin["C"], vin["D"], vin["init"], dy=dy, dfinal=dfinal)
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}
    base = {k: vin[k] for k in keys}
    for k in keys:
        V = rng.standard_normal(base[k].shape)
        h = 1e-6 * max(1.0, float(np.max(np.abs(base[k]))))
        fd = (J(dict(base, **{k: base[k] + h * V})) - J(dict(base, **{k: base[k] - h * V}))) / (2 * h)
        an = float(np.sum(g[names[k]] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, fd, an)
    # the empty sequence's dinit is its dfinal
    assert np.array_equal(g["dinit"][1], dfinal[1])


def test_vjp_exact_on_the_linear_inputs():
    """Exact identities, no finite differences: the scan is jointly linear in
    (x, init) with every other input fixed, linear in B when init and D are
    absent, linear in C (with no final-state term and no D) and its D term is
    D x.  For a map linear in an input u, J(u) = <dJ/du, u>, so:
      J = <dx, x> + <dinit, init>            (all inputs present)
      J = <dB, B>                            (no init, no D)
      sum(dy * y) = <dC, C>                  (no D, dfinal = 0)
      dD_h = sum over b, t, p of x * dy      (the D term alone)
    A dropped term, a wrong sign or a transposed index in any of the four
    gradients breaks its identity far beyond rounding."""
    inp, dy, dfinal = problem(2, 23, 4, 3, 5, 2, seed=41)

    def rel(a, b):
        return abs(a - b) / max(abs(a), abs(b), 1e-300)

    g = oracle.scan_vjp(**inp, dy=dy, dfinal=dfinal)
    j = J(inp, dy, dfinal)
    assert rel(j, float(np.sum(g["dx"] * inp["x"]) + np.sum(g["dinit"] * inp["init"]))) < 1e-11

    lin = dict(inp, init=None, D=None)
    g = oracle.scan_vjp(**lin, dy=dy, dfinal=dfinal)
    assert rel(J(lin, dy, dfinal), float(np.sum(g["dB"] * lin["B"]))) < 1e-11

    y, _ = oracle.scan(**dict(inp, D=None))
    g = oracle.scan_vjp(**dict(inp, D=None), dy=dy, dfinal=None)
    assert rel(float(np.sum(dy * y)), float(np.sum(g["dC"] * inp["C"]))) < 1e-11

    g = oracle.scan_vjp(**inp, dy=dy, dfinal=dfinal)
    assert np.allclose(g["dD"], np.einsum("blhp,blhp->h", inp["x"], dy), rtol=1e-12, atol=1e-12)
