"""GPU parity of the prefill scan (through the C ABI) against the CPU oracle.

Element-by-element at sizes the oracle finishes in seconds (several chunks and
a ragged tail), per stage against the fp64 chunked form, and at the full
workload sizes on sampled (batch, head) pairs that the oracle computes one by
one.  Bars: 1e-4 (fp32 x/B/C) and 2e-2 (bf16 x/B/C) in the rel_err metric.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.chunked import chunked_scan
import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import synth

from helpers import TOL, f64, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(inp, chunk, **kw):
    d = to_dev(inp, DEV)
    y, fin = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=chunk,
                          init_state=d["init"], **kw)
    torch.cuda.synchronize()
    return y, fin


def check_full(inp, chunk, dtype):
    y, fin = run_gpu(inp, chunk)
    yo, fo = oracle.scan(**oracle_args(inp))
    ey, ef = rel_err(f64(y), yo), rel_err(f64(fin), fo)
    print(f"  rel_err y {ey:.3e} final {ef:.3e} (bar {TOL[dtype]:.0e})", flush=True)
    assert ey <= TOL[dtype], f"y rel err {ey:.3e}"
    assert ef <= TOL[dtype], f"final rel err {ef:.3e}"
    return ey, ef


@pytest.mark.parametrize("name", ["tiny_f32", "m130m_bf16"])
def test_workload_full(name):
    spec = synth.WORKLOADS[name]
    announce(f"scan_fwd {name}")
    inp = synth.scan_inputs(spec)
    dtype = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    check_full(inp, spec.chunk, dtype)


def sampled_check(inp, chunk, pairs, dtype):
    y, fin = run_gpu(inp, chunk)
    ref = oracle.scan_heads(inp, pairs)
    yg = torch.stack([y[b, :, h] for b, h in pairs]).float().cpu().numpy()
    fg = torch.stack([fin[b, h] for b, h in pairs]).cpu().numpy()
    yo = np.stack([ref[p][0] for p in pairs])
    fo = np.stack([ref[p][1] for p in pairs])
    ey, ef = rel_err(yg, yo), rel_err(fg, fo)
    print(f"  rel_err y {ey:.3e} final {ef:.3e} (bar {TOL[dtype]:.0e})", flush=True)
    assert ey <= TOL[dtype], f"y rel err {ey:.3e}"
    assert ef <= TOL[dtype], f"final rel err {ef:.3e}"


def test_workload_2p7b_sampled():
    spec = synth.WORKLOADS["m2p7b_bf16"]
    announce(f"scan_fwd {spec.name} sampled heads")
    inp = synth.scan_inputs(spec)
    sampled_check(inp, spec.chunk, [(0, 0), (0, 17), (0, 41), (0, 63), (0, 79)],
                  torch.bfloat16)


def test_workload_batched_long_sampled():
    spec = synth.WORKLOADS["batched_long_bf16"]
    announce(f"scan_fwd {spec.name} sampled (batch, head)")
    inp = synth.scan_inputs(spec)
    sampled_check(inp, spec.chunk, [(0, 0), (3, 37), (5, 50), (7, 79)], torch.bfloat16)


SHAPES = [
    # Bt, L, H, P, N, G, chunk, dtype
    (1, 256, 4, 16, 16, 1, 64, "f32"),
    (2, 300, 4, 8, 32, 2, 64, "f32"),        # ragged tail
    (1, 100, 2, 5, 4, 1, 16, "f32"),         # odd headdim, tiny dstate
    (1, 77, 3, 7, 8, 3, 32, "bf16"),
    (2, 513, 4, 64, 128, 2, 256, "bf16"),    # ragged, MFMA-sized heads
    (1, 640, 6, 64, 64, 3, 128, "bf16"),
    (1, 384, 2, 64, 128, 1, 64, "bf16"),
    (1, 200, 2, 64, 128, 2, 128, "f32"),
    (3, 96, 4, 32, 256, 4, 32, "bf16"),
    (1, 100, 3, 64, 64, 1, 256, "bf16"),     # one partial chunk: half its row tiles empty
    (2, 33, 2, 64, 128, 2, 64, "bf16"),      # 33 tokens: a one-row second tile
    (1, 70, 2, 256, 256, 1, 32, "f32"),      # the largest headdim and d_state accepted
    (2, 50, 4, 8, 4, 2, 16, "bf16"),         # the smallest d_state and chunk accepted
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("with_init", [True, False])
def test_shapes_full(shape, with_init):
    Bt, L, H, P, N, G, chunk, dt_ = shape
    announce(f"scan_fwd shape {shape} init={with_init}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk, dt_, dt_rule="ranged",
                             init="normal" if with_init else "zero", seed=SHAPES.index(shape))
    inp = synth.scan_inputs(spec)
    check_full(inp, chunk, torch.bfloat16 if dt_ == "bf16" else torch.float32)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_chunk_sizes_agree_with_oracle(chunk):
    announce(f"chunk invariance chunk={chunk}")
    spec = synth.custom_spec(1, 512, 4, 64, 128, 1, chunk, "bf16", dt_rule="ranged",
                             init="normal", seed=5)
    inp = synth.scan_inputs(spec)
    check_full(inp, chunk, torch.bfloat16)


def test_no_D_no_final():
    announce("D=None, final not requested")
    spec = synth.custom_spec(1, 130, 2, 16, 16, 1, 64, "f32", init="normal", seed=9)
    inp = synth.scan_inputs(spec)
    inp["D"] = None
    y, fin = run_gpu(inp, 64, return_final_state=False)
    assert fin is None
    yo, _ = oracle.scan(**oracle_args(inp))
    assert rel_err(f64(y), yo) <= TOL[torch.float32]


def test_final_state_in_place():
    announce("final_state aliases init_state")
    spec = synth.custom_spec(2, 200, 4, 64, 128, 2, 64, "bf16", dt_rule="ranged",
                             init="normal", seed=10)
    inp = synth.scan_inputs(spec)
    d = to_dev(inp, DEV)
    h = d["init"].clone()
    y, fin = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=64,
                          init_state=h, final_state=h)
    torch.cuda.synchronize()
    assert fin.data_ptr() == h.data_ptr()
    yo, fo = oracle.scan(**oracle_args(inp))
    assert rel_err(f64(y), yo) <= TOL[torch.bfloat16]
    assert rel_err(f64(h), fo) <= TOL[torch.bfloat16]


def test_empty_sequence():
    announce("seqlen 0")
    spec = synth.custom_spec(2, 0, 4, 16, 16, 1, 64, "f32", init="normal", seed=11)
    inp = synth.scan_inputs(spec)
    y, fin = run_gpu(inp, 64)
    assert y.shape[1] == 0
    assert torch.equal(fin.cpu(), inp["init"])
    inp["init"] = None
    y, fin = run_gpu(inp, 64)
    assert torch.count_nonzero(fin).item() == 0


def test_split_resume_matches_oracle():
    announce("split/resume through final_state")
    spec = synth.custom_spec(1, 700, 4, 64, 128, 1, 256, "bf16", dt_rule="ranged",
                             init="normal", seed=12)
    inp = synth.scan_inputs(spec)
    d = to_dev(inp, DEV)
    k = 333
    y1, f1 = ssd.scan_fwd(d["x"][:, :k].contiguous(), d["dt"][:, :k].contiguous(), d["A"],
                          d["B"][:, :k].contiguous(), d["C"][:, :k].contiguous(), d["D"],
                          chunk=256, init_state=d["init"])
    y2, f2 = ssd.scan_fwd(d["x"][:, k:].contiguous(), d["dt"][:, k:].contiguous(), d["A"],
                          d["B"][:, k:].contiguous(), d["C"][:, k:].contiguous(), d["D"],
                          chunk=256, init_state=f1)
    torch.cuda.synchronize()
    yo, fo = oracle.scan(**oracle_args(inp))
    assert rel_err(np.concatenate([f64(y1), f64(y2)], axis=1), yo) <= TOL[torch.bfloat16]
    assert rel_err(f64(f2), fo) <= TOL[torch.bfloat16]


def test_deterministic():
    announce("run-to-run bitwise determinism")
    spec = synth.custom_spec(2, 1000, 8, 64, 128, 2, 256, "bf16", dt_rule="ranged",
                             init="normal", seed=13)
    inp = synth.scan_inputs(spec)
    y1, f1 = run_gpu(inp, 256)
    y2, f2 = run_gpu(inp, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


# ------------------------------------------------------------ stage parity
@pytest.mark.parametrize("shape", [
    (1, 256, 4, 16, 16, 1, 64, "f32"),
    (2, 300, 4, 64, 128, 2, 128, "bf16"),
    (1, 520, 3, 64, 64, 1, 256, "bf16"),
    (2, 150, 6, 32, 32, 3, 32, "bf16"),      # generic kernels: groups, ragged tail
])
def test_stages_against_chunked_form(shape):
    Bt, L, H, P, N, G, chunk, dt_ = shape
    announce(f"stages {shape}")
    dtype = torch.bfloat16 if dt_ == "bf16" else torch.float32
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk, dt_, dt_rule="ranged", init="normal",
                             seed=14)
    inp = synth.scan_inputs(spec)
    ref = chunked_scan(**oracle_args(inp), chunk=chunk)
    d = to_dev(inp, DEV)
    like = (d["x"], d["B"])
    Acs = ssd.chunk_cumsum(d["dt"], d["A"], chunk, like)
    torch.cuda.synchronize()
    # fp32 cumsum of fp32 products: absolute error relative to the running magnitude
    assert np.max(np.abs(f64(Acs) - ref["Acs"])) <= 1e-5 * max(1.0, np.max(np.abs(ref["Acs"])))
    S = ssd.chunk_state(d["x"], d["B"], d["dt"], Acs, chunk)
    torch.cuda.synchronize()
    assert rel_err(f64(S), ref["S"]) <= TOL[dtype]
    fin = ssd.state_passing(S, Acs, chunk, like, init_state=d["init"])
    torch.cuda.synchronize()
    assert rel_err(f64(S), ref["Hin"]) <= TOL[dtype]
    assert rel_err(f64(fin), ref["final"]) <= TOL[dtype]
    y = ssd.chunk_scan(d["x"], d["dt"], d["B"], d["C"], d["D"], Acs, S, chunk)
    torch.cuda.synchronize()
    assert rel_err(f64(y), ref["y"]) <= TOL[dtype]


def test_golden_fixture_on_gpu():
    import json
    import os
    announce("golden tiny fixture")
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "tiny_f32_oracle.json")))
    inp = synth.scan_inputs(synth.WORKLOADS[doc["workload"]])
    y, fin = run_gpu(inp, synth.WORKLOADS[doc["workload"]].chunk)
    yv = f64(y)
    got = np.array([yv[tuple(i)] for i, _ in doc["y"]])
    ref = np.array([v for _, v in doc["y"]])
    assert rel_err(got, ref) <= TOL[torch.float32]


def test_fwd_repeats_bit_for_bit():
    """Run-to-run determinism at the 2.7B head shape: no atomics and fixed
    reduction orders in the forward, so two calls on the same inputs (one
    with a fresh workspace, one reusing the first call's) agree bit for bit."""
    spec = synth.WORKLOADS["m2p7b_bf16"]
    announce(f"scan_fwd {spec.name} twice, bit for bit")
    d = to_dev(synth.scan_inputs(spec), DEV)
    ws = torch.empty(ssd.workspace_size(spec.batch, spec.seqlen, spec.nheads, spec.headdim,
                                        spec.dstate, spec.ngroups, spec.chunk, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    outs = []
    for w in (None, ws, ws):
        y, fin = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=spec.chunk,
                              init_state=d["init"], workspace=w)
        outs.append((y, fin))
    torch.cuda.synchronize()
    for y, fin in outs[1:]:
        assert torch.equal(y, outs[0][0])
        assert torch.equal(fin, outs[0][1])
