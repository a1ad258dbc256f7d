"""The elementwise edges around the scan in a Mamba block, in fp64
(TEST INFRASTRUCTURE ONLY: tests, smoke() and the bench's CPU leg).

The pyshine "Mamba" repository tour ("Why You Need This") describes them:
the block feeds the scan softplus(dt + dt_bias), where the bias is set so that
softplus(bias) starts between dt_min and dt_max, and the scan kernels can gate
their output with z.  The pages give the gate's name, not its formula; the
reading taken here is the Mamba gate y * silu(z), silu(z) = z * sigmoid(z).
The clamp to [dt_min, dt_max] is the reading of "dt limits" that makes that
range hold after training moves the bias.

Each function is the plain definition, written out.
"""
from __future__ import annotations

import numpy as np

from . import f64


def softplus(v):
    """log(1 + e^v), evaluated as log(e^0 + e^v) without overflow."""
    return np.logaddexp(0.0, f64(v))


def dt_activation(dt, bias=None, softplus_on: bool = False, limit=None):
    """The step size the scan uses: (dt + bias), then softplus when
    ``softplus_on``, then a clamp to ``limit`` = (lo, hi) when given.  dt is
    [..., nheads]; bias [nheads] broadcasts over the leading axes."""
    d = f64(dt)
    if bias is not None:
        d = d + f64(bias)
    if softplus_on:
        d = softplus(d)
    if limit is not None:
        d = np.clip(d, float(limit[0]), float(limit[1]))
    return d


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z)."""
    z = f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gate(y, z):
    """The gated output y * silu(z)."""
    return f64(y) * silu(z)


def gated_rmsnorm(y, z, weight, eps: float, groups: int):
    """Gated RMSNorm of a scan output, the step that the pyshine tour of the
    Mamba repository (Mamba2 in the block walk-through) says replaces the
    plain output activation.  The page names the module and gives no formula;
    the reading taken is the gate first, then a root-mean-square
    normalisation over channel groups, then a per-channel weight:

        v   = y * silu(z)            (v = y when z is None)
        out = v / sqrt(mean(v^2 over the group) + eps) * weight

    y, z: [..., nheads, headdim]; weight: [nheads * headdim]; the channels of
    a token, in (head, headdim) order, split into ``groups`` equal groups of
    whole heads."""
    v = f64(y) if z is None else gate(y, z)
    shape = v.shape
    H, P = shape[-2], shape[-1]
    if H % groups:
        raise ValueError("groups must divide nheads")
    g = v.reshape(shape[:-2] + (groups, (H // groups) * P))
    ms = np.mean(g * g, axis=-1, keepdims=True)
    out = g / np.sqrt(ms + float(eps))
    return out.reshape(shape) * f64(weight).reshape(H, P)
