"""CPU oracle for the SSD scan and decode step (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it, and the
two share no code.

* :func:`scan` / :func:`step` wrap the fp64 token-by-token recurrence in
  ``ssd_oracle.c`` (the definition of the operation).
* :func:`scan_vjp` is the gradient of the scan (adjoint recurrence, fp64).
* :func:`scan_varlen` runs a packed ragged batch sequence by sequence.
* :mod:`oracle.edges` holds the fp64 dt activation and output gate.
* :mod:`oracle.chunked` is an fp64 numpy version of the chunked algorithm
  (per-chunk matrix form plus a scan of chunk states), used to check the
  recurrence and to give per-stage values.

Every function takes numpy arrays or CPU torch tensors of any float dtype and
converts them to float64 exactly (bf16 and fp32 values are representable).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIB names another build of ssd_oracle.c to load instead (the
# sanitizer test runs the pins against an ASan/UBSan build this way)
_LIB_PATH = os.environ.get("SSD_ORACLE_LIB") or os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build() -> str:
    """Compile ssd_oracle.c with gcc (no fast-math, no FMA contraction, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-ffp-contract=off",
        "-fno-fast-math", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm",
    ])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ssd_oracle_scan.argtypes = [_I64] * 6 + [_D] * 9 + [ctypes.c_int]
        lib.ssd_oracle_scan.restype = ctypes.c_int
        lib.ssd_oracle_step.argtypes = [_I64] * 5 + [_D] * 8 + [ctypes.c_int]
        lib.ssd_oracle_step.restype = ctypes.c_int
        lib.ssd_oracle_scan_vjp.argtypes = [_I64] * 6 + [_D] * 16 + [ctypes.c_int]
        lib.ssd_oracle_scan_vjp.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.argtypes = []
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def f64(a) -> np.ndarray | None:
    """Exact conversion of a numpy array or CPU torch tensor to contiguous float64."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def max_threads() -> int:
    return _load().ssd_oracle_max_threads()


def scan(x, dt, A, B, C, D=None, init=None, nthreads: int = 0):
    """fp64 recurrence over the whole sequence.  Returns (y, final_state)."""
    x, dt, A, B, C, D, init = (f64(v) for v in (x, dt, A, B, C, D, init))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bt, L, H) and A.shape == (H,)
    assert B.shape == (Bt, L, G, N) and C.shape == B.shape
    assert D is None or D.shape == (H,)
    assert init is None or init.shape == (Bt, H, P, N)
    y = np.empty((Bt, L, H, P))
    final = np.empty((Bt, H, P, N))
    rc = _load().ssd_oracle_scan(Bt, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(init), _ptr(y), _ptr(final),
                                 int(nthreads))
    if rc == -2:
        raise MemoryError("oracle: the per-thread state rows could not be allocated")
    if rc != 0:
        raise ValueError("oracle: invalid shape")
    return y, final


def step(state, x, dt, A, B, C, D=None, nthreads: int = 0):
    """One fp64 decode step.  Returns (y, new_state); the input state is not modified."""
    s = f64(state).copy()
    x, dt, A, B, C, D = (f64(v) for v in (x, dt, A, B, C, D))
    Bt, H, P, N = s.shape
    G = B.shape[1]
    assert x.shape == (Bt, H, P) and dt.shape == (Bt, H) and A.shape == (H,)
    assert B.shape == (Bt, G, N) and C.shape == B.shape
    y = np.empty((Bt, H, P))
    rc = _load().ssd_oracle_step(Bt, H, P, N, G, _ptr(s), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle: invalid shape")
    return y, s


def scan_heads(inputs: dict, pairs, nthreads: int = 0):
    """Recurrence for selected (batch, head) pairs only.

    ``inputs`` holds x, dt, A, B, C, D, init as produced for the full problem.
    Returns {(b, h): (y [L,P], final [P,N])}.  Each pair is an independent
    one-head problem, so sampled checks at large sizes stay cheap.
    """
    x, B = inputs["x"], inputs["B"]
    H, G = x.shape[2], B.shape[2]
    R = H // G
    out = {}
    for b, h in pairs:
        g = h // R
        init = inputs.get("init")
        y, fin = scan(
            x[b:b + 1, :, h:h + 1, :], inputs["dt"][b:b + 1, :, h:h + 1],
            inputs["A"][h:h + 1], B[b:b + 1, :, g:g + 1, :], inputs["C"][b:b + 1, :, g:g + 1, :],
            None if inputs.get("D") is None else inputs["D"][h:h + 1],
            None if init is None else init[b:b + 1, h:h + 1],
            nthreads=nthreads)
        out[(b, h)] = (y[0, :, 0, :], fin[0, 0])
    return out


def scan_varlen(cu_seqlens, x, dt, A, B, C, D=None, init=None, nthreads: int = 0):
    """A ragged batch: sequence s is tokens [cu[s], cu[s+1]) of the packed
    x [total, H, P], dt [total, H], B/C [total, G, N], each run through
    :func:`scan` on its own from init[s] (zero when init is None).  Returns
    (y [total, H, P], finals [nseq, H, P, N])."""
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    x, dt, B, C = f64(x), f64(dt), f64(B), f64(C)
    init = f64(init)
    nseq = len(cu) - 1
    H, P = x.shape[1], x.shape[2]
    N = B.shape[2]
    y = np.zeros_like(x)
    finals = np.zeros((nseq, H, P, N))
    for s in range(nseq):
        a, b = cu[s], cu[s + 1]
        h0 = None if init is None else init[s:s + 1]
        if b == a:
            finals[s] = 0.0 if h0 is None else h0[0]
            continue
        ys, fs = scan(x[None, a:b], dt[None, a:b], A, B[None, a:b], C[None, a:b], D, h0,
                      nthreads=nthreads)
        y[a:b] = ys[0]
        finals[s] = fs[0]
    return y, finals


def scan_vjp(x, dt, A, B, C, D=None, init=None, dy=None, dfinal=None, nthreads: int = 0) -> dict:
    """Gradients of J = sum(dy * y) + sum(dfinal * final_state) with respect to
    x, dt, A, B, C, D and init, by the adjoint recurrence in ssd_oracle.c.
    dy is required; dfinal may be None (no final-state term).  Returns a dict
    of float64 arrays: dx, ddt, dA, dB, dC, dD, dinit."""
    x, dt, A, B, C, D, init, dy, dfinal = (f64(v) for v in (x, dt, A, B, C, D, init, dy, dfinal))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape and (dfinal is None or dfinal.shape == (Bt, H, P, N))
    out = {"dx": np.empty_like(x), "ddt": np.empty((Bt, L, H)), "dA": np.empty(H),
           "dB": np.empty((Bt, L, G, N)), "dC": np.empty((Bt, L, G, N)), "dD": np.empty(H),
           "dinit": np.empty((Bt, H, P, N))}
    rc = _load().ssd_oracle_scan_vjp(
        Bt, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
        _ptr(dy), _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle vjp failed ({rc})")
    return out


def scan_vjp_edges(x, dt_raw, A, B, C, D=None, init=None, dy=None, dfinal=None, dt_bias=None,
                   dt_softplus: bool = False, dt_limit=None, z=None, norm_weight=None,
                   norm_eps: float = 1e-5, norm_groups: int = 1, nthreads: int = 0) -> dict:
    """Gradients of J = sum(dy * y) + sum(dfinal * final_state) for the scan
    with its fused edges: dt = edges.dt_activation(dt_raw, dt_bias,
    dt_softplus, dt_limit) is the step size, and the output is gated,
    y = scan(...) * silu(z), when z is given.  This is the chain rule over
    scan_vjp:
      - dy reaches the scan as dy * silu(z);
      - dz = dy * y_scan * silu'(z), with silu'(z) = s (1 + z (1 - s)) and
        s = sigmoid(z);
      - ddt (with respect to dt_raw) = ddt_scan * d dt / d dt_raw, where the
        derivative is sigmoid(dt_raw + bias) with softplus on (1 without),
        times 0 where the clamp holds the value at a bound it was pushed past;
      - ddt_bias = ddt summed over batch and tokens.
    With ``norm_weight``, the output is edges.gated_rmsnorm(y, z, norm_weight,
    norm_eps, norm_groups) instead: per token and group, with v the gated
    output, r = 1 / sqrt(mean(v^2) + eps) and S = sum(dy w v) over the group's
    CG channels, the gradient reaching v is dv = r (w dy - v r^2 S / CG), and
    dnorm_weight = dy v r summed over the leading axes; the gate's rule above
    then applies with dv in place of dy.
    Returns scan_vjp's dict with ddt replaced, plus dz (z given), ddt_bias
    (dt_bias given) and dnorm_weight (norm_weight given)."""
    from . import edges
    dt = edges.dt_activation(dt_raw, dt_bias, dt_softplus, dt_limit)
    dy = f64(dy)
    extra = {}
    if z is not None or norm_weight is not None:
        y, _ = scan(x, dt, A, B, C, D, init, nthreads=nthreads)
    if norm_weight is not None:
        v = y if z is None else edges.gate(y, z)
        shape = v.shape
        H, P = shape[-2], shape[-1]
        CG = (H // norm_groups) * P
        gshape = shape[:-2] + (norm_groups, CG)
        vg, dg = v.reshape(gshape), dy.reshape(gshape)
        wg = f64(norm_weight).reshape(norm_groups, CG)
        r = 1.0 / np.sqrt(np.mean(vg * vg, axis=-1, keepdims=True) + float(norm_eps))
        S = np.sum(dg * wg * vg, axis=-1, keepdims=True)
        dv = r * (wg * dg - vg * r * r * S / CG)
        extra["dnorm_weight"] = np.sum(dg * vg * r, axis=tuple(range(len(gshape) - 2))).reshape(-1)
        dy = dv.reshape(shape)
    if z is not None:
        zz = f64(z)
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-zz))
        dz = dy * y * (sg * (1.0 + zz * (1.0 - sg)))
        dy_scan = dy * edges.silu(zz)
    else:
        dy_scan = dy
    g = scan_vjp(x, dt, A, B, C, D, init, dy_scan, dfinal, nthreads=nthreads)
    u = f64(dt_raw) + (0.0 if dt_bias is None else f64(dt_bias))
    if dt_softplus:
        with np.errstate(over="ignore"):
            dact = 1.0 / (1.0 + np.exp(-u))
    else:
        dact = np.ones_like(u)
    if dt_limit is not None:
        pre = edges.softplus(u) if dt_softplus else u
        dact = dact * ((pre >= float(dt_limit[0])) & (pre <= float(dt_limit[1])))
    g["ddt"] = g["ddt"] * dact
    if dt_bias is not None:
        g["ddt_bias"] = g["ddt"].sum(axis=tuple(range(g["ddt"].ndim - 1)))
    if z is not None:
        g["dz"] = dz
    g.update(extra)
    return g


def scan_vjp_varlen(cu_seqlens, x, dt, A, B, C, D=None, init=None, dy=None, dfinal=None,
                    nthreads: int = 0) -> dict:
    """Gradients for a ragged batch (scan_varlen): every sequence's own
    scan_vjp on its tokens (a sequence sees no other's tokens, starts from its
    init and ends in its final state).  dx, ddt, dB, dC are per packed token,
    dinit per sequence, dA and dD summed over the sequences."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    x, dt, B, C, dy = f64(x), f64(dt), f64(B), f64(C), f64(dy)
    total, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    ns = len(cu) - 1
    out = {"dx": np.zeros_like(x), "ddt": np.zeros((total, H)), "dA": np.zeros(H),
           "dB": np.zeros((total, G, N)), "dC": np.zeros((total, G, N)), "dD": np.zeros(H),
           "dinit": np.zeros((ns, H, P, N))}
    for s in range(ns):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            if dfinal is not None:
                out["dinit"][s] = f64(dfinal)[s]
            continue
        g = scan_vjp(x[None, a:b], dt[None, a:b], A, B[None, a:b], C[None, a:b], D,
                     None if init is None else f64(init)[s:s + 1], dy[None, a:b],
                     None if dfinal is None else f64(dfinal)[s:s + 1], nthreads=nthreads)
        out["dx"][a:b] = g["dx"][0]
        out["ddt"][a:b] = g["ddt"][0]
        out["dB"][a:b] = g["dB"][0]
        out["dC"][a:b] = g["dC"][0]
        out["dinit"][s] = g["dinit"][0]
        out["dA"] += g["dA"]
        out["dD"] += g["dD"]
    return out
