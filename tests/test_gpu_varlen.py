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
from mamba_ssd_chunked_scan_amd import binding, synth

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
    # last chunks ending at, before and after the 32-row tiles and the
    # 64-token stage pairs (short chunks skip their empty stages, output
    # rows and C.B row tiles)
    "mfma_tile_bounds": ([32, 64, 95, 96, 97, 160, 224, 225, 288, 287], 4, 64, 64, 1, 256,
                         "bf16"),
    "mfma_q128_tails": ([31, 32, 33, 96, 97, 127, 192, 193, 0, 5], 4, 64, 128, 1, 128, "bf16"),
    "generic_f32": ([0, 17, 64, 65, 150, 1, 90], 4, 16, 16, 2, 64, "f32"),
    "generic_bf16_p32": ([5, 128, 129, 0, 300], 4, 32, 32, 2, 128, "bf16"),
}


def _dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def _run(d, chunk, edges=False, **kw):
    """ssd_scan_fwd_varlen on device inputs; on calls that hand states between
    blocks, also checks that every hand-off wait completed."""
    e = {}
    if edges:
        e = dict(dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=LIMIT, z=d["gate"])
    total, H, P = d["x"].shape
    G, N = d["B"].shape[1], d["B"].shape[2]
    nseq = d["cu_seqlens"].numel() - 1
    io = binding.SSD_BF16 if d["x"].dtype == torch.bfloat16 else binding.SSD_F32
    ws = torch.empty(max(binding.varlen_workspace_size(nseq, total, H, P, N, G, chunk,
                                                       d["x"].dtype), 1),
                     dtype=torch.uint8, device=DEV)
    y, fin = ssd.scan_fwd_varlen(d["x"], d["dt_raw"] if edges else d["dt"], d["A"], d["B"],
                                 d["C"], d["cu_seqlens"], d["D"], chunk=chunk,
                                 init_states=d["init"], workspace=ws, **e, **kw)
    torch.cuda.synchronize()
    desc = binding.VarlenDesc(nseq, total, H, P, N, G, chunk, io, 0)
    err = binding.error_word(ws, desc, varlen=True)
    assert err in (None, 0), f"a hand-off wait ran out (error word {err})"
    return y, fin


@pytest.mark.parametrize("path", ["separate", "chained", "fused"])
@pytest.mark.parametrize("edges", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_varlen_vs_oracle(name, edges, path, monkeypatch):
    lengths, H, P, N, G, Q, dt_ = CASES[name]
    if path == "fused" and Q != 256:
        pytest.skip("the single-kernel path covers chunk 256 only")
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    announce(f"varlen {name} edges={edges} path={path}")
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


@pytest.mark.parametrize("path", ["separate", "chained"])
def test_varlen_final_in_place(path, monkeypatch):
    """final_states may be init_states in a ragged call too, empty sequences
    included (their final state is their initial one)."""
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    lengths, H, P, N, G, Q, dt_ = CASES["mfma_edges"]
    announce(f"varlen final in place path={path}")
    inp = synth.varlen_inputs(lengths, H, P, N, G, dt_, seed=45)
    d = _dev(inp)
    h = d["init"].clone()
    y, fin = ssd.scan_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"],
                                 d["D"], chunk=Q, init_states=h, final_states=h)
    torch.cuda.synchronize()
    assert fin.data_ptr() == h.data_ptr()
    yo, fo = oracle.scan_varlen(inp["cu_seqlens"], inp["x"], inp["dt"], inp["A"], inp["B"],
                                inp["C"], inp["D"], inp["init"])
    assert rel_err(f64(y), yo) <= TOL[inp["x"].dtype]
    assert rel_err(f64(h), fo) <= TOL[inp["x"].dtype]


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


@pytest.mark.parametrize("path", ["separate", "chained"])
def test_sequence_past_2gib(path, monkeypatch):
    """A ragged batch whose second sequence (333 tokens) starts past byte
    2^31 of the packed x: 2,097,300 + 333 tokens x 8 heads of headdim 64,
    inputs drawn on the device.  The oracle checks the second sequence whole
    (y and final state) and the first 333 tokens of the first one."""
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    lens = [2_097_300, 333]
    total, H, P, N, G, Q = sum(lens), 8, 64, 128, 1, 256
    print(f"[case] varlen {lens} x {H} heads, past 2 GiB, path={path}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(63)
    bf = torch.bfloat16
    d = {
        "x": torch.randn((total, H, P), generator=gen, device=DEV, dtype=bf),
        "B": torch.randn((total, G, N), generator=gen, device=DEV, dtype=bf),
        "C": torch.randn((total, G, N), generator=gen, device=DEV, dtype=bf),
        "dt": torch.rand((total, H), generator=gen, device=DEV) * 0.099 + 0.001,
        "A": -torch.exp(torch.rand((H,), generator=gen, device=DEV) * float(np.log(16.0))),
        "D": torch.randn((H,), generator=gen, device=DEV),
        "init": torch.randn((len(lens), H, P, N), generator=gen, device=DEV) * 0.1,
        "cu_seqlens": torch.tensor([0, lens[0], total], dtype=torch.int32, device=DEV),
    }
    assert lens[0] * H * P * 2 > (1 << 31)
    y, fin = _run(d, Q)
    for s, (t0, n) in enumerate([(lens[0], lens[1]), (0, 333)]):
        sl = slice(t0, t0 + n)
        cpu = {k: d[k][sl].cpu().unsqueeze(0) for k in ("x", "dt", "B", "C")}
        yo, fo = oracle.scan(cpu["x"], cpu["dt"], d["A"].cpu(), cpu["B"], cpu["C"],
                             d["D"].cpu(), d["init"][1 - s:2 - s].cpu())
        assert rel_err(f64(y[sl].unsqueeze(0)), yo) <= TOL[bf], s
        if s == 0:  # the second sequence, whole
            assert rel_err(f64(fin[1:2]), fo) <= TOL[bf]
    del d, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["separate", "chained", "fused"])
def test_serving_mix_2p7b_sampled(path, monkeypatch):
    """32 requests of log-uniform length in [16, 4096] at the 2.7B head shape
    (80 heads), in the launch configuration the bench times; 8 sampled
    (sequence, head) pairs against the oracle one by one."""
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    lengths = synth.serving_lengths(32, seed=7)
    announce(f"varlen serving mix total={sum(lengths)} path={path}")
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


BWD_CASES = {
    # lengths cross the gradient's 64-token chunks: 63 / 64 / 65, one token, empty
    "bwd_mfma": ([64, 63, 0, 65, 1, 200, 130], 4, 64, 128, 2, "bf16"),
    "bwd_mfma_n64": ([5, 0, 129, 64], 6, 64, 64, 2, "bf16"),
    "bwd_generic_f32": ([0, 17, 33, 32, 90, 1], 4, 16, 16, 2, "f32"),
}


def _ragged_grads(name, seed):
    lengths, H, P, N, G, dt_ = BWD_CASES[name]
    vin = synth.varlen_inputs(lengths, H, P, N, G, dt_, seed=seed)
    rng = np.random.default_rng(seed + 1)
    io = torch.bfloat16 if dt_ == "bf16" else torch.float32
    dy = torch.from_numpy(rng.standard_normal(tuple(vin["x"].shape), dtype=np.float32)).to(io)
    dfin = torch.from_numpy(rng.standard_normal(tuple(vin["init"].shape), dtype=np.float32))
    return vin, dy, dfin, io


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_varlen_bwd_vs_oracle(name):
    """ssd_scan_bwd_varlen against the per-sequence fp64 adjoint (itself
    pinned by finite differences of the ragged forward oracle)."""
    announce(f"varlen bwd {name}")
    vin, dy, dfin, io = _ragged_grads(name, seed=81)
    d = _dev(vin)
    g = ssd.scan_bwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"],
                            dy.to(DEV), d["D"], chunk=64, init_states=d["init"],
                            dfinal_states=dfin.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.scan_vjp_varlen(vin["cu_seqlens"], vin["x"], vin["dt"], vin["A"], vin["B"],
                                 vin["C"], vin["D"], vin["init"], dy=dy, dfinal=dfin)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit"):
        e = rel_err(f64(g[k]), ref[k])
        assert e <= TOL[io], (k, e)


@pytest.mark.parametrize("name", ["bwd_mfma", "bwd_generic_f32"])
def test_varlen_bwd_edges_vs_oracle(name):
    """The ragged gradient with every edge (dt bias, softplus, clamp, gate):
    each sequence against oracle.scan_vjp_edges on its own tokens; dt_bias's
    gradient summed over the sequences."""
    announce(f"varlen bwd edges {name}")
    vin, dy, dfin, io = _ragged_grads(name, seed=83)
    lim = (1e-3, 0.05)
    d = _dev(vin)
    g = ssd.scan_bwd_varlen(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["cu_seqlens"],
                            dy.to(DEV), d["D"], chunk=64, init_states=d["init"],
                            dfinal_states=dfin.to(DEV), dt_bias=d["dt_bias"], dt_softplus=True,
                            dt_limit=lim, z=d["gate"])
    torch.cuda.synchronize()
    cu = vin["cu_seqlens"].numpy()
    H = vin["A"].shape[0]
    ref = {k: np.zeros(tuple(vin[s].shape)) for k, s in
           (("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dz", "x"),
            ("dinit", "init"))}
    ref.update(dA=np.zeros(H), dD=np.zeros(H), ddt_bias=np.zeros(H))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            ref["dinit"][s] = dfin[s].double().numpy()
            continue
        r = oracle.scan_vjp_edges(vin["x"][None, a:b], vin["dt_raw"][None, a:b], vin["A"],
                                  vin["B"][None, a:b], vin["C"][None, a:b], vin["D"],
                                  vin["init"][s:s + 1], dy=dy[None, a:b], dfinal=dfin[s:s + 1],
                                  dt_bias=vin["dt_bias"], dt_softplus=True, dt_limit=lim,
                                  z=vin["gate"][None, a:b])
        for k in ("dx", "ddt", "dB", "dC", "dz"):
            ref[k][a:b] = r[k][0]
        ref["dinit"][s] = r["dinit"][0]
        for k in ("dA", "dD", "ddt_bias"):
            ref[k] += r[k]
    for k in ref:
        e = rel_err(f64(g[k]), ref[k])
        assert e <= TOL[io], (k, e)
