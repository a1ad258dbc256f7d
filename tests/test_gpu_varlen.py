"""GPU parity of the variable-length (ragged) prefill against the oracle's
sequence-by-sequence driver, and its equivalences with the fixed-length call.

Lengths include the cases the chunking has to get right: empty sequences,
one token, one short of a chunk, a chunk, one past, several chunks with a
ragged tail.  Bars as for the plain scan."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import edges as oe
import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import synth

from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIMIT = (1e-3, 0.1)


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


# name: (lengths, H, P, N, G, chunk, dtype)
CASES = {
    "mfma_edges": ([0, 1, 255, 256, 257, 700, 3, 0, 512, 33], 8, 64, 128, 2, 256, "bf16"),
    "mfma_q64_n64": ([64, 63, 65, 1, 200, 0, 130], 4, 64, 64, 1, 64, "bf16"),
    "generic_f32": ([0, 17, 64, 65, 150, 1, 90], 4, 16, 16, 2, 64, "f32"),
    "generic_bf16_p32": ([5, 128, 129, 0, 300], 4, 32, 32, 2, 128, "bf16"),
}


def _dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def _run(d, chunk, edges=False, **kw):
    e = {}
    if edges:
        e = dict(dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=LIMIT, z=d["gate"])
    y, fin = ssd.scan_fwd_varlen(d["x"], d["dt_raw"] if edges else d["dt"], d["A"], d["B"],
                                 d["C"], d["cu_seqlens"], d["D"], chunk=chunk,
                                 init_states=d["init"], **e, **kw)
    torch.cuda.synchronize()
    return y, fin


@pytest.mark.parametrize("edges", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_varlen_vs_oracle(name, edges):
    lengths, H, P, N, G, Q, dt_ = CASES[name]
    announce(f"varlen {name} edges={edges}")
    inp = synth.varlen_inputs(lengths, H, P, N, G, dt_, seed=41)
    y, fin = _run(_dev(inp), Q, edges)
    dt = (oe.dt_activation(inp["dt_raw"], inp["dt_bias"], True, LIMIT) if edges else inp["dt"])
    yo, fo = oracle.scan_varlen(inp["cu_seqlens"], inp["x"], dt, inp["A"], inp["B"], inp["C"],
                                inp["D"], inp["init"])
    if edges:
        yo = oe.gate(yo, inp["gate"])
    tol = TOL[inp["x"].dtype]
    assert rel_err(f64(y), yo) <= tol
    assert rel_err(f64(fin), fo) <= tol
    # empty sequences pass their init state through exactly
    for s, n in enumerate(lengths):
        if n == 0:
            assert torch.equal(fin[s].cpu(), inp["init"][s])


@pytest.mark.parametrize("Bt,L,H,P,N,G,Q,dt_", [
    (3, 700, 8, 64, 128, 2, 256, "bf16"),   # MFMA path
    (2, 333, 4, 16, 16, 2, 64, "f32"),      # generic path
])
def test_equal_lengths_equal_batched_call(Bt, L, H, P, N, G, Q, dt_):
    """Equal lengths, packed, are the batch layout: bit for bit the batched
    call (same chunk boundaries, same kernels)."""
    announce(f"varlen == batched {Bt}x{L}")
    inp = _dev(synth.varlen_inputs([L] * Bt, H, P, N, G, dt_, seed=42))
    y, fin = _run(inp, Q)
    yb, fb = ssd.scan_fwd(inp["x"].view(Bt, L, H, P), inp["dt"].view(Bt, L, H), inp["A"],
                          inp["B"].view(Bt, L, G, N), inp["C"].view(Bt, L, G, N), inp["D"],
                          chunk=Q, init_state=inp["init"])
    torch.cuda.synchronize()
    assert torch.equal(y, yb.view(y.shape)) and torch.equal(fin, fb)


def test_serving_mix_2p7b_sampled():
    """32 requests of log-uniform length in [16, 4096] at the 2.7B head shape
    (80 heads), in the launch configuration the bench times; 8 sampled
    (sequence, head) pairs against the oracle one by one."""
    lengths = synth.serving_lengths(32, seed=7)
    announce(f"varlen serving mix total={sum(lengths)}")
    inp = synth.varlen_inputs(lengths, 80, 64, 128, 1, "bf16", seed=43)
    y, fin = _run(_dev(inp), 256)
    cu = inp["cu_seqlens"].tolist()
    rng = np.random.default_rng(3)
    for s, h in zip(rng.choice(32, 8, replace=False), rng.choice(80, 8)):
        a, b = cu[s], cu[s + 1]
        yo, fo = oracle.scan(inp["x"][None, a:b, h:h + 1], inp["dt"][None, a:b, h:h + 1],
                             inp["A"][h:h + 1], inp["B"][None, a:b], inp["C"][None, a:b],
                             inp["D"][h:h + 1], inp["init"][s:s + 1, h:h + 1])
        assert rel_err(f64(y[a:b, h]), yo[0, :, 0]) <= TOL[torch.bfloat16], (s, h)
        assert rel_err(f64(fin[s, h]), fo[0, 0]) <= TOL[torch.bfloat16], (s, h)


def test_graph_replay_with_new_lengths():
    """The chunk table is built on the device, so one captured call serves any
    split of the same token count: rewrite cu_seqlens in place, replay, and
    get the eager result for the new lengths, bit for bit."""
    announce("varlen graph replay")
    splits = [[100, 300, 0, 624], [1024, 0, 0, 0], [1, 1, 1, 1021], [256, 256, 256, 256]]
    inp = _dev(synth.varlen_inputs(splits[0], 8, 64, 128, 2, "bf16", seed=44))
    total = sum(splits[0])
    ws = torch.empty(ssd.varlen_workspace_size(4, total, 8, 64, 128, 2, 256, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty_like(inp["x"])
    fin = torch.empty((4, 8, 64, 128), device=DEV)
    cu = inp["cu_seqlens"]
    call = lambda yy, ff: ssd.scan_fwd_varlen(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                              cu, inp["D"], chunk=256, init_states=inp["init"],
                                              workspace=ws, y=yy, final_states=ff)
    call(y, fin)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y, fin)
    for lens in splits[1:] + splits[:1]:
        cu.copy_(torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32))
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        ye, fe = torch.empty_like(y), torch.empty_like(fin)
        call(ye, fe)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(fin, fe), lens
