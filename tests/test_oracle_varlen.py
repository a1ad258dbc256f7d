"""Pins for the oracle's ragged-batch driver: what a packed batch of
independent sequences must satisfy, each checked against the batched oracle
or against a perturbation, not against the driver itself."""
import numpy as np

import oracle
from mamba_ssd_chunked_scan_amd import synth


def packed(Bt, L, H, P, N, G, seed):
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=16, dtype="f32", init="normal", seed=seed)
    inp = synth.scan_inputs(spec)
    flat = {k: oracle.f64(inp[k]) for k in ("x", "dt", "B", "C")}
    return inp, {k: v.reshape((Bt * L,) + v.shape[2:]) for k, v in flat.items()}


def test_equal_lengths_is_the_batched_scan():
    """Sequences of equal length, packed, are a batch laid out the same way."""
    inp, pk = packed(3, 40, 2, 4, 8, 1, seed=5)
    cu = np.arange(4) * 40
    y, fin = oracle.scan_varlen(cu, pk["x"], pk["dt"], inp["A"], pk["B"], pk["C"], inp["D"],
                                inp["init"])
    yb, fb = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init"])
    assert np.array_equal(y, yb.reshape(y.shape)) and np.array_equal(fin, fb)


def test_sequences_are_independent():
    """Changing one sequence's tokens changes nothing in the others: the state
    resets at every boundary."""
    inp, pk = packed(1, 90, 2, 4, 8, 2, seed=6)
    cu = np.array([0, 17, 17, 50, 90])   # includes an empty sequence
    init = np.random.default_rng(0).standard_normal((4, 2, 4, 8))
    y0, f0 = oracle.scan_varlen(cu, pk["x"], pk["dt"], inp["A"], pk["B"], pk["C"], inp["D"], init)
    x2 = pk["x"].copy()
    x2[17:50] += 1.0                     # sequence 2 only
    y1, f1 = oracle.scan_varlen(cu, x2, pk["dt"], inp["A"], pk["B"], pk["C"], inp["D"], init)
    same = np.r_[0:17, 50:90]
    assert np.array_equal(y0[same], y1[same])
    assert np.array_equal(f0[[0, 1, 3]], f1[[0, 1, 3]])
    assert not np.array_equal(f0[2], f1[2])
    # the empty sequence passes its init state through
    assert np.array_equal(f0[1], init[1])


def test_sequence_equals_a_slice_with_its_own_state():
    """A sequence inside a packed batch equals that token range scanned alone."""
    inp, pk = packed(1, 64, 2, 4, 8, 1, seed=7)
    cu = np.array([0, 23, 64])
    init = np.random.default_rng(1).standard_normal((2, 2, 4, 8))
    y, fin = oracle.scan_varlen(cu, pk["x"], pk["dt"], inp["A"], pk["B"], pk["C"], inp["D"], init)
    ys, fs = oracle.scan(pk["x"][None, 23:], pk["dt"][None, 23:], inp["A"], pk["B"][None, 23:],
                         pk["C"][None, 23:], inp["D"], init[1:2])
    assert np.array_equal(y[23:], ys[0]) and np.array_equal(fin[1], fs[0])
