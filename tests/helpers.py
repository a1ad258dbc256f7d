"""Shared helpers for the GPU parity tests."""
import numpy as np
import torch

# Parity bars: max relative error with an rms floor (see rel_err), 1e-4 when
# x/B/C are fp32 and 2e-2 when they are bf16 with fp32 accumulation.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

INPUT_KEYS = ("x", "dt", "A", "B", "C", "D", "init")


def rel_err(got, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)).

    A plain per-element ratio is unbounded where the reference crosses zero;
    the rms of the reference is the floor of the denominator.
    """
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), max(rms, 1e-300))
    return float(np.max(np.abs(g - o) / den))


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def to_dev(inp: dict, dev="cuda:0") -> dict:
    return {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}


def oracle_args(inp: dict) -> dict:
    return {k: inp[k] for k in INPUT_KEYS}
