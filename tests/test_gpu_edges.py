"""GPU parity of the fused scan edges (dt bias + softplus + clamp applied in
the kernels, output gate y * silu(z) applied before the output rounding)
against the fp64 oracle: oracle.edges applied around the oracle recurrence.

Inputs are the raw edge inputs of the generator: dt before activation, the
per-head bias softplus^-1(dt0), a N(0, 1) gate.  Bars as for the plain scan.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import edges as oe
import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import binding, synth

from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIMIT = (1e-3, 0.1)


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


SPECS = {
    # MFMA path (bf16, headdim 64): several chunks and a ragged tail
    "mfma_q256_n128": synth.custom_spec(2, 700, 8, 64, 128, 2, chunk=256, dtype="bf16",
                                        dt_rule="ranged", init="normal", seed=21),
    "mfma_q64_n64": synth.custom_spec(1, 300, 4, 64, 64, 1, chunk=64, dtype="bf16",
                                      dt_rule="ranged", init="normal", seed=22),
    # generic fp32 path
    "generic_f32": synth.custom_spec(1, 333, 4, 16, 16, 2, chunk=64, dtype="f32",
                                     dt_rule="ranged", init="normal", seed=23),
}


def _run(spec, which, inp):
    use_dt = which in ("all", "dt")
    use_gate = which in ("all", "gate")
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    kw = {}
    if use_dt:
        kw.update(dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=LIMIT)
    if use_gate:
        kw["z"] = d["gate"]
    x = d["x"]
    ws = torch.empty(max(ssd.workspace_size(x.shape[0], x.shape[1], x.shape[2], x.shape[3],
                                            d["B"].shape[3], d["B"].shape[2], spec.chunk,
                                            x.dtype), 1),
                     dtype=torch.uint8, device=DEV)
    y, fin = ssd.scan_fwd(x, d["dt_raw"] if use_dt else d["dt"], d["A"], d["B"], d["C"],
                          d["D"], chunk=spec.chunk, init_state=d["init"], workspace=ws, **kw)
    torch.cuda.synchronize()
    # every hand-off wait of the call completed (None: the call has none)
    err = binding.error_word(ws, binding._scan_desc(x, d["B"], spec.chunk))
    assert err in (None, 0), f"a hand-off wait ran out (error word {err})"
    return y, fin


def _reference(inp, which):
    use_dt = which in ("all", "dt")
    dt = (oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT) if use_dt
          else inp["dt"])
    yo, fo = oracle.scan(inp["x"], dt, inp["A"], inp["B"], inp["C"], inp["D"], inp["init"])
    if which in ("all", "gate"):
        yo = oe.gate(yo, inp["gate"])
    return yo, fo


@pytest.mark.parametrize("path", ["separate", "chained", "fused"])
@pytest.mark.parametrize("which", ["all", "dt", "gate"])
@pytest.mark.parametrize("name", list(SPECS))
def test_scan_edges_vs_oracle(name, which, path, monkeypatch):
    spec = SPECS[name]
    if path == "fused" and spec.chunk != 256:
        pytest.skip("the single-kernel path covers chunk 256 only")
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    announce(f"scan edges {name} {which} path={path}")
    inp = synth.scan_edge_inputs(spec)
    y, fin = _run(spec, which, inp)
    yo, fo = _reference(inp, which)
    tol = TOL[inp["x"].dtype]
    assert rel_err(f64(y), yo) <= tol
    assert rel_err(f64(fin), fo) <= tol


@pytest.mark.parametrize("name", list(SPECS))
def test_zero_bias_equals_plain_call(name):
    """A zero bias activates the edge path (the first kernel writes the
    activated dt to the workspace and the later ones read it) without
    changing a value: results are bit for bit those of the plain call."""
    spec = SPECS[name]
    announce(f"zero bias {name}")
    inp = synth.scan_edge_inputs(spec)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
    y0, f0 = ssd.scan_fwd(*args, chunk=spec.chunk, init_state=d["init"])
    y1, f1 = ssd.scan_fwd(*args, chunk=spec.chunk, init_state=d["init"],
                          dt_bias=torch.zeros_like(d["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


def test_edges_at_bench_workload_sampled():
    """The 2.7B prefill workload (batch 1, 4096 tokens, 80 heads) with every
    edge on, in the bench's launch configuration; 6 sampled heads against the
    oracle one by one."""
    spec = synth.WORKLOADS["m2p7b_bf16"]
    announce("scan edges m2p7b sampled")
    inp = synth.scan_edge_inputs(spec)
    y, fin = _run(spec, "all", inp)
    dt = oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT)
    ref_in = dict(inp, dt=torch.from_numpy(dt))
    heads = [0, 13, 31, 47, 64, 79]
    ref = oracle.scan_heads(ref_in, [(0, h) for h in heads])
    for h in heads:
        yo, fo = ref[(0, h)]
        yo = oe.gate(yo, inp["gate"][0, :, h])
        assert rel_err(f64(y[0, :, h]), yo) <= TOL[torch.bfloat16], h
        assert rel_err(f64(fin[0, h]), fo) <= TOL[torch.bfloat16], h


@pytest.mark.parametrize("shape", [
    # Bt, T, H, P, N, G, dtype  (LDS-staged and register-prefetch multi-step kernels)
    (2, 20, 8, 64, 128, 2, torch.bfloat16),
    (3, 5, 4, 12, 32, 1, torch.float32),
])
def test_step_edges(shape):
    """Decode with every edge on: ssd_step_ex against the oracle step, and
    ssd_step_multi_ex bit for bit equal to the chained single steps."""
    Bt, T, H, P, N, G, dtype = shape
    announce(f"step edges {shape}")
    dn = "bf16" if dtype == torch.bfloat16 else "f32"
    inp = synth.edge_decode_inputs(Bt, T, H, P, N, G, dn, seed=31 + T)
    d = {k: v.to(DEV) for k, v in inp.items()}
    ekw = dict(dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=LIMIT)
    s_chain = d["state"].clone()
    ys = []
    for t in range(T):
        ys.append(ssd.step(s_chain, d["x"][:, t].clone(), d["dt_raw"][:, t].clone(), d["A"],
                           d["B"][:, t].clone(), d["C"][:, t].clone(), d["D"],
                           z=d["gate"][:, t].clone(), **ekw))
    y_chain = torch.stack(ys, 1)
    s_multi = d["state"].clone()
    y_multi = ssd.step_multi(s_multi, d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"],
                             z=d["gate"], **ekw)
    torch.cuda.synchronize()
    assert torch.equal(y_multi, y_chain)
    assert torch.equal(s_multi, s_chain)
    # oracle: activated dt, the recurrence token by token, then the gate
    dt = oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT)
    s = inp["state"]
    yo = []
    for t in range(T):
        yt, s = oracle.step(s, inp["x"][:, t], dt[:, t], inp["A"], inp["B"][:, t],
                            inp["C"][:, t], inp["D"])
        yo.append(oe.gate(yt, inp["gate"][:, t]))
    assert rel_err(f64(y_chain), np.stack(yo, 1)) <= TOL[dtype]
    assert rel_err(f64(s_chain), s) <= TOL[dtype]


def _norm_weight(H, P, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(1.0 + 0.5 * rng.standard_normal(H * P)).float()


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("name,groups", [("mfma_q256_n128", 0), ("mfma_q64_n64", 2),
                                         ("generic_f32", 1)])
def test_scan_gated_rmsnorm(name, groups, gated):
    """Every edge on plus the gated RMSNorm pass (norm_groups 0 = the B/C
    groups, 2, and 1 = the whole row), against the oracle scan followed by
    oracle.edges.gated_rmsnorm; and the norm without a gate."""
    spec = SPECS[name]
    announce(f"scan gated norm {name} groups {groups} gated {gated}")
    inp = synth.scan_edge_inputs(spec)
    H, P = spec.nheads, spec.headdim
    w = _norm_weight(H, P, seed=41)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y, fin = ssd.scan_fwd(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], chunk=spec.chunk,
                          init_state=d["init"], dt_bias=d["dt_bias"], dt_softplus=True,
                          dt_limit=LIMIT, z=d["gate"] if gated else None,
                          norm_weight=w.to(DEV), norm_eps=1e-5, norm_groups=groups)
    torch.cuda.synchronize()
    dt = oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT)
    yo, fo = oracle.scan(inp["x"], dt, inp["A"], inp["B"], inp["C"], inp["D"], inp["init"])
    ng = groups or spec.ngroups
    yo = oe.gated_rmsnorm(yo, inp["gate"] if gated else None, w, 1e-5, ng)
    tol = TOL[inp["x"].dtype]
    assert rel_err(f64(y), yo) <= tol
    assert rel_err(f64(fin), fo) <= tol


def test_varlen_gated_rmsnorm():
    """The norm pass over a ragged batch: every packed token normalised, as
    for each sequence alone."""
    announce("varlen gated norm")
    lengths = [37, 0, 130, 64]
    H, P, N, G = 4, 64, 64, 2
    vin = synth.varlen_inputs(lengths, H, P, N, G, "bf16", seed=44)
    d = {k: v.to(DEV) for k, v in vin.items()}
    w = _norm_weight(H, P, seed=45)
    y, fin = ssd.scan_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"],
                                 d["D"], chunk=64, init_states=d["init"], z=d["gate"],
                                 norm_weight=w.to(DEV), norm_eps=1e-5)
    torch.cuda.synchronize()
    yo, fo = oracle.scan_varlen(vin["cu_seqlens"], vin["x"], vin["dt"], vin["A"], vin["B"],
                                vin["C"], vin["D"], vin["init"])
    yo = oe.gated_rmsnorm(yo, vin["gate"], w, 1e-5, G)
    assert rel_err(f64(y), yo) <= TOL[torch.bfloat16]
    assert rel_err(f64(fin), fo) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("shape", [
    (2, 6, 8, 64, 128, 2, torch.bfloat16),
    (3, 4, 4, 12, 32, 1, torch.float32),
])
def test_step_gated_rmsnorm(shape):
    """Decode with the gate and the norm pass: ssd_step_ex against the oracle
    step, and ssd_step_multi_ex bit for bit equal to the chained steps."""
    Bt, T, H, P, N, G, dtype = shape
    announce(f"step gated norm {shape}")
    dn = "bf16" if dtype == torch.bfloat16 else "f32"
    inp = synth.edge_decode_inputs(Bt, T, H, P, N, G, dn, seed=51 + T)
    d = {k: v.to(DEV) for k, v in inp.items()}
    w = _norm_weight(H, P, seed=52)
    nkw = dict(dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=LIMIT, norm_weight=w.to(DEV),
               norm_eps=1e-5)
    s_chain = d["state"].clone()
    ys = []
    for t in range(T):
        ys.append(ssd.step(s_chain, d["x"][:, t].clone(), d["dt_raw"][:, t].clone(), d["A"],
                           d["B"][:, t].clone(), d["C"][:, t].clone(), d["D"],
                           z=d["gate"][:, t].clone(), **nkw))
    y_chain = torch.stack(ys, 1)
    s_multi = d["state"].clone()
    y_multi = ssd.step_multi(s_multi, d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"],
                             z=d["gate"], **nkw)
    torch.cuda.synchronize()
    assert torch.equal(y_multi, y_chain)
    assert torch.equal(s_multi, s_chain)
    dt = oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT)
    s = inp["state"]
    yo = []
    for t in range(T):
        yt, s = oracle.step(s, inp["x"][:, t], dt[:, t], inp["A"], inp["B"][:, t],
                            inp["C"][:, t], inp["D"])
        yo.append(oe.gated_rmsnorm(yt, inp["gate"][:, t], w, 1e-5, G))
    assert rel_err(f64(y_chain), np.stack(yo, 1)) <= TOL[dtype]
    assert rel_err(f64(s_chain), s) <= TOL[dtype]
