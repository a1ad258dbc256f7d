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
