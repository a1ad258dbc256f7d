"""Seeded synthetic inputs for the SSD chunked scan and the cached decode step.

This module only draws random numbers and rounds them to the storage dtype. It
holds none of the scan's arithmetic, which is why both the CPU oracle and the
HIP path may take their inputs from it.

Shapes are the Mamba-2 head shapes: headdim 64 and d_state 128, with 24 heads
(d_model 768, expand 2) for the 130M model and 80 heads (d_model 2560, expand 2)
for the 2.7B model, as the pyshine "Mamba" repository tour lists them
(overview list; "From Install to a Running Block"). Prompt lengths follow the
prefill sweep of "Compiler-First State Space Duality and Portable O(1)
Autoregressive Caching for Inference" (paperlayer summary, A.2 Benchmark
Configurations) and the chunk size of 256 its §3 ("Chunked recurrence") uses.

Value recipes (synthetic stand-ins for real activations, no checkpoint needed):
  x, B, C ~ N(0, 1), drawn in fp32 and rounded to nearest even when bf16;
  A_h = -exp(u_h), u_h ~ U(0, ln 16)      (A is a negative scalar per head);
  D_h ~ N(0, 1);
  dt, rule "shifted":  softplus(z - 4), z ~ N(0, 1);
  dt, rule "ranged":   clamp(softplus(z + bias_h), 1e-3, 0.1) with
                       bias_h = softplus^-1(dt0_h), dt0_h = exp(U(ln 1e-3, ln 0.1)),
                       the dt_min/dt_max initialisation the repository tour
                       describes ("Why You Need This");
  init state ~ N(0, 0.1) (standard deviation 0.1) or zero.
Draw order is fixed: x, B, C, z, u, D, dt0, init.

For the fused scan edges (dt bias, softplus and clamp applied inside the
kernels, output gate silu(g)), scan_edge_inputs hands over the raw values
instead of the activated dt: dt_raw = z, dt_bias_h = softplus^-1(dt0_h), and a
gate g ~ N(0, 1) of x's shape, drawn after init.  Which activation to apply is
the caller's business; this module applies none to them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "ScanSpec", "DecodeSpec", "WORKLOADS", "DECODE_WORKLOADS", "scan_inputs",
    "DecodeStream", "custom_spec", "scan_edge_inputs", "edge_decode_inputs", "varlen_inputs",
    "serving_lengths",
]


@dataclasses.dataclass(frozen=True)
class ScanSpec:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str          # storage dtype of x, B, C and y: "f32" or "bf16"
    dt_rule: str        # "shifted" or "ranged"
    init: str           # "zero" or "normal"
    seed: int

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    steps: int
    dtype: str
    seed: int


WORKLOADS = {
    s.name: s for s in [
        ScanSpec("tiny_f32", 1, 256, 4, 16, 16, 1, 64, "f32", "shifted", "zero", 1),
        ScanSpec("m130m_bf16", 1, 2048, 24, 64, 128, 1, 256, "bf16", "ranged", "zero", 2),
        ScanSpec("m2p7b_bf16", 1, 4096, 80, 64, 128, 1, 256, "bf16", "ranged", "normal", 3),
        ScanSpec("batched_long_bf16", 8, 16384, 80, 64, 128, 8, 256, "bf16", "ranged",
                 "normal", 4),
    ]
}

DECODE_WORKLOADS = {
    s.name: s for s in [
        DecodeSpec("decode_2p7b_b1", 1, 80, 64, 128, 1, 4096, "bf16", 5),
        DecodeSpec("decode_2p7b_b64", 64, 80, 64, 128, 1, 4096, "bf16", 5),
    ]
}


def custom_spec(batch, seqlen, nheads, headdim, dstate, ngroups=1, chunk=64, dtype="f32",
                dt_rule="shifted", init="normal", seed=0, name="custom") -> ScanSpec:
    return ScanSpec(name, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                    dt_rule, init, seed)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def _storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _dt(rng_z: np.ndarray, rule: str, dt0: np.ndarray | None) -> np.ndarray:
    z = rng_z.astype(np.float64)
    if rule == "shifted":
        v = _softplus(z - 4.0)
    elif rule == "ranged":
        bias = np.log(np.expm1(dt0))          # softplus^-1(dt0)
        v = np.clip(_softplus(z + bias), 1e-3, 0.1)
    else:
        raise ValueError(f"unknown dt rule {rule!r}")
    return v.astype(np.float32)


def scan_inputs(spec: ScanSpec, seed: int | None = None) -> dict:
    """CPU tensors for one prefill call: x, dt, A, B, C, D, init (None when zero)."""
    return _scan_draw(spec, seed)[0]


def scan_edge_inputs(spec: ScanSpec, seed: int | None = None) -> dict:
    """scan_inputs plus the raw edge inputs: dt_raw [B, L, H] fp32 (the z of
    the dt recipe, before any bias or activation), dt_bias [H] fp32 =
    softplus^-1(dt0), and gate [B, L, H, P] in the storage dtype."""
    out, rng, z, dt0 = _scan_draw(spec, seed)
    g = rng.standard_normal((spec.batch, spec.seqlen, spec.nheads, spec.headdim),
                            dtype=np.float32)
    out["dt_raw"] = torch.from_numpy(z)
    out["dt_bias"] = torch.from_numpy(np.log(np.expm1(dt0)).astype(np.float32))
    out["gate"] = _storage(g, spec.dtype)
    return out


def edge_decode_inputs(batch, nsteps, nheads, headdim, dstate, ngroups, dtype, seed) -> dict:
    """Raw inputs of nsteps decode tokens with fused edges, prefill layout:
    state, x, dt_raw, A, B, C, D, dt_bias, gate (the recipes above)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    H, P, N = nheads, headdim, dstate
    u = rng.uniform(0.0, math.log(16.0), size=H)
    D = rng.standard_normal(H)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=H))
    state = rng.standard_normal((batch, H, P, N), dtype=np.float32) * np.float32(0.1)
    x = rng.standard_normal((batch, nsteps, H, P), dtype=np.float32)
    Bm = rng.standard_normal((batch, nsteps, ngroups, N), dtype=np.float32)
    Cm = rng.standard_normal((batch, nsteps, ngroups, N), dtype=np.float32)
    z = rng.standard_normal((batch, nsteps, H), dtype=np.float32)
    g = rng.standard_normal((batch, nsteps, H, P), dtype=np.float32)
    return {
        "state": torch.from_numpy(state),
        "x": _storage(x, dtype),
        "dt_raw": torch.from_numpy(z),
        "A": torch.from_numpy((-np.exp(u)).astype(np.float32)),
        "B": _storage(Bm, dtype),
        "C": _storage(Cm, dtype),
        "D": torch.from_numpy(D.astype(np.float32)),
        "dt_bias": torch.from_numpy(np.log(np.expm1(dt0)).astype(np.float32)),
        "gate": _storage(g, dtype),
    }


def serving_lengths(nseq: int, seed: int, lo: int = 16, hi: int = 4096) -> list[int]:
    """Lengths of a ragged serving batch: log-uniform integers in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(v) for v in np.exp(rng.uniform(math.log(lo), math.log(hi + 1), size=nseq))]


def varlen_inputs(lengths, nheads, headdim, dstate, ngroups, dtype, seed) -> dict:
    """A packed ragged batch with the recipes above (dt rule "ranged", init
    ~ N(0, 0.1) per sequence), plus the raw edge inputs: cu_seqlens int32
    [nseq + 1], x [total, H, P], dt and dt_raw [total, H], B, C [total, G, N],
    A, D, dt_bias [H], init [nseq, H, P, N], gate [total, H, P].
    Draw order: x, B, C, z, u, D, dt0, init, gate."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(v) for v in lengths]
    total, nseq = sum(lengths), len(lengths)
    H, P, N, G = nheads, headdim, dstate, ngroups
    x = rng.standard_normal((total, H, P), dtype=np.float32)
    Bm = rng.standard_normal((total, G, N), dtype=np.float32)
    Cm = rng.standard_normal((total, G, N), dtype=np.float32)
    z = rng.standard_normal((total, H), dtype=np.float32)
    u = rng.uniform(0.0, math.log(16.0), size=H)
    D = rng.standard_normal(H)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=H))
    init = rng.standard_normal((nseq, H, P, N), dtype=np.float32) * np.float32(0.1)
    g = rng.standard_normal((total, H, P), dtype=np.float32)
    return {
        "cu_seqlens": torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32),
        "x": _storage(x, dtype),
        "dt": torch.from_numpy(_dt(z, "ranged", dt0)),
        "dt_raw": torch.from_numpy(z),
        "A": torch.from_numpy((-np.exp(u)).astype(np.float32)),
        "B": _storage(Bm, dtype),
        "C": _storage(Cm, dtype),
        "D": torch.from_numpy(D.astype(np.float32)),
        "dt_bias": torch.from_numpy(np.log(np.expm1(dt0)).astype(np.float32)),
        "init": torch.from_numpy(init),
        "gate": _storage(g, dtype),
    }


def _scan_draw(spec: ScanSpec, seed: int | None):
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    Bt, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    x = rng.standard_normal((Bt, L, H, P), dtype=np.float32)
    Bm = rng.standard_normal((Bt, L, G, N), dtype=np.float32)
    Cm = rng.standard_normal((Bt, L, G, N), dtype=np.float32)
    z = rng.standard_normal((Bt, L, H), dtype=np.float32)
    u = rng.uniform(0.0, math.log(16.0), size=H)
    D = rng.standard_normal(H)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=H))
    init = None
    if spec.init == "normal":
        init = torch.from_numpy(
            (rng.standard_normal((Bt, H, P, N), dtype=np.float32) * np.float32(0.1)))
    elif spec.init != "zero":
        raise ValueError(f"unknown init {spec.init!r}")
    return {
        "x": _storage(x, spec.dtype),
        "dt": torch.from_numpy(_dt(z, spec.dt_rule, dt0)),
        "A": torch.from_numpy((-np.exp(u)).astype(np.float32)),
        "B": _storage(Bm, spec.dtype),
        "C": _storage(Cm, spec.dtype),
        "D": torch.from_numpy(D.astype(np.float32)),
        "init": init,
    }, rng, z, dt0


class DecodeStream:
    """Fixed A, D and initial state, then a fresh (x, dt, B, C) per decode step.

    Draw order: u (A), D, dt0, state, then per step x, B, C, z.
    """

    def __init__(self, spec: DecodeSpec, seed: int | None = None):
        self.spec = spec
        self.rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
        H, P, N = spec.nheads, spec.headdim, spec.dstate
        u = self.rng.uniform(0.0, math.log(16.0), size=H)
        D = self.rng.standard_normal(H)
        self.dt0 = np.exp(self.rng.uniform(math.log(1e-3), math.log(0.1), size=H))
        self.A = torch.from_numpy((-np.exp(u)).astype(np.float32))
        self.D = torch.from_numpy(D.astype(np.float32))
        self.state = torch.from_numpy(
            self.rng.standard_normal((spec.batch, H, P, N), dtype=np.float32) * np.float32(0.1))

    def next_step(self) -> dict:
        s, rng = self.spec, self.rng
        x = rng.standard_normal((s.batch, s.nheads, s.headdim), dtype=np.float32)
        Bm = rng.standard_normal((s.batch, s.ngroups, s.dstate), dtype=np.float32)
        Cm = rng.standard_normal((s.batch, s.ngroups, s.dstate), dtype=np.float32)
        z = rng.standard_normal((s.batch, s.nheads), dtype=np.float32)
        return {
            "x": _storage(x, s.dtype),
            "dt": torch.from_numpy(_dt(z, "ranged", self.dt0)),
            "B": _storage(Bm, s.dtype),
            "C": _storage(Cm, s.dtype),
        }
