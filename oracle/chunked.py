"""fp64 chunked form of the SSD scan (TEST INFRASTRUCTURE ONLY).

This follows the chunked algorithm as "Compiler-First State Space Duality and
Portable O(1) Autoregressive Caching for Inference" (paperlayer summary)
describes it: inside each fixed-size chunk the output is a parallel matrix
computation, and a light sequential scan carries one summary state from chunk to
chunk (§3 Method, "Chunked recurrence"); the causal structure is a fixed
lower-triangular mask (§3, "Primitive-level implementation"); the work is three
contractions: the intra-chunk output, the accumulation of each chunk's state,
and the inter-chunk state update (B.5, last paragraph).

Per chunk c (tokens t0 .. t0+q-1, q <= chunk; the last chunk may be short), per
batch row b and head h with a = A[h]:

  Acs[i]     = sum_{k <= i} dt[t0+k] * a             (inclusive, restarts per chunk)
  M[i, j]    = (C_i . B_j) * exp(Acs[i] - Acs[j]) * dt_j   for j <= i, else 0
  y_diag[i]  = sum_j M[i, j] * x_j
  y_off[i]   = exp(Acs[i]) * (C_i . H_c)                 (H_c: state entering chunk c)
  y[i]       = y_diag[i] + y_off[i] + D * x_i
  S_c        = sum_j exp(Acs[q-1] - Acs[j]) * dt_j * x_j (outer) B_j
  H_{c+1}    = exp(Acs[q-1]) * H_c + S_c,   H_0 = init state (or 0)

Written with numpy einsum over whole chunks in float64; the only loop is the
sequential one over chunks.  It shares no code with the recurrence in
ssd_oracle.c, so agreement between the two checks both.
"""
from __future__ import annotations

import numpy as np

from . import f64


def chunked_scan(x, dt, A, B, C, D=None, init=None, chunk: int = 256) -> dict:
    """Returns a dict with y, final and the per-stage arrays.

    Stage arrays (T = number of chunks):
      Acs   [Bt, H, L]          within-chunk inclusive cumsum of dt*A
      S     [Bt, T, H, P, N]    state contributed by each chunk alone
      Hin   [Bt, T, H, P, N]    state entering each chunk
      y_diag, y_off [Bt, L, H, P]
    """
    x, dt, A, B, C, D, init = (f64(v) for v in (x, dt, A, B, C, D, init))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    R = H // G
    assert H % G == 0 and chunk >= 1
    Bh = np.repeat(B, R, axis=2)            # group of head h is h // R
    Ch = np.repeat(C, R, axis=2)
    T = -(-L // chunk)
    Hc = np.zeros((Bt, H, P, N)) if init is None else init.copy()
    Dv = np.zeros(H) if D is None else D
    y = np.empty((Bt, L, H, P))
    y_diag = np.empty_like(y)
    y_off = np.empty_like(y)
    Acs_all = np.empty((Bt, H, L))
    S_all = np.empty((Bt, T, H, P, N))
    Hin_all = np.empty((Bt, T, H, P, N))
    for c in range(T):
        t0, t1 = c * chunk, min(L, (c + 1) * chunk)
        q = t1 - t0
        xc, dtc, Bc, Cc = x[:, t0:t1], dt[:, t0:t1], Bh[:, t0:t1], Ch[:, t0:t1]
        acs = np.cumsum(dtc * A[None, None, :], axis=1)                 # [Bt, q, H]
        seg = acs[:, :, None, :] - acs[:, None, :, :]                    # [Bt, i, j, H]
        causal = np.tril(np.ones((q, q), dtype=bool))[None, :, :, None]
        decay = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
        CB = np.einsum("bihn,bjhn->bijh", Cc, Bc)
        M = CB * decay * dtc[:, None, :, :]
        yd = np.einsum("bijh,bjhp->bihp", M, xc)
        yo = np.einsum("bih,bihn,bhpn->bihp", np.exp(acs), Cc, Hc)
        y_diag[:, t0:t1] = yd
        y_off[:, t0:t1] = yo
        y[:, t0:t1] = yd + yo + Dv[None, None, :, None] * xc
        w = np.exp(acs[:, -1:, :] - acs) * dtc                            # [Bt, q, H]
        S = np.einsum("bjh,bjhp,bjhn->bhpn", w, xc, Bc)
        Acs_all[:, :, t0:t1] = acs.transpose(0, 2, 1)
        S_all[:, c] = S
        Hin_all[:, c] = Hc
        Hc = np.exp(acs[:, -1, :])[:, :, None, None] * Hc + S
    return {"y": y, "final": Hc, "Acs": Acs_all, "S": S_all, "Hin": Hin_all,
            "y_diag": y_diag, "y_off": y_off}
