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
from mamba_ssd_chunked_scan_amd import binding, synth

from helpers import TOL, f64, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(inp, chunk, **kw):
    """ssd_scan_fwd on the device copies of inp; on calls that hand states
    between blocks (the chained state pass or the single-kernel path), also
    checks that every hand-off wait completed."""
    d = to_dev(inp, DEV)
    x = d["x"]
    ws = torch.empty(max(ssd.workspace_size(x.shape[0], x.shape[1], x.shape[2], x.shape[3],
                                            d["B"].shape[3], d["B"].shape[2], chunk, x.dtype), 1),
                     dtype=torch.uint8, device=DEV)
    y, fin = ssd.scan_fwd(x, d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=chunk,
                          init_state=d["init"], workspace=ws, **kw)
    torch.cuda.synchronize()
    err = binding.error_word(ws, binding._scan_desc(x, d["B"], chunk))
    assert err in (None, 0), f"a hand-off wait ran out (error word {err})"
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


@pytest.mark.parametrize("path", ["auto", "chained"])
def test_workload_2p7b_full(path, monkeypatch):
    """The 2.7B head shape prefill (4096 tokens, 80 heads): every element of y
    and of the final state against the oracle."""
    if path == "chained":
        monkeypatch.setenv("SSD_PREFILL_PATH", "chained")
    spec = synth.WORKLOADS["m2p7b_bf16"]
    announce(f"scan_fwd {spec.name} all heads path={path}")
    check_full(synth.scan_inputs(spec), spec.chunk, torch.bfloat16)


def test_workload_2p7b_f32_sampled():
    """The same shape with fp32 x/B/C (the generic kernels): sampled heads."""
    spec = synth.custom_spec(1, 4096, 80, 64, 128, 1, 256, "f32", dt_rule="ranged",
                             init="normal", seed=3, name="m2p7b_f32")
    announce(f"scan_fwd {spec.name} sampled heads")
    sampled_check(synth.scan_inputs(spec), spec.chunk, [(0, 0), (0, 33), (0, 79)],
                  torch.float32)


@pytest.mark.parametrize("path", ["auto", "separate"])
def test_workload_batched_long_rows(path, monkeypatch):
    """The batched long prefill (8 x 16384 tokens, 8 groups): every head of
    batch rows 0 and 7, each row's oracle run on its own (the oracle holds one
    row at a time).  The automatic choice chains the state pass here."""
    if path == "separate":
        monkeypatch.setenv("SSD_PREFILL_PATH", "separate")
    spec = synth.WORKLOADS["batched_long_bf16"]
    announce(f"scan_fwd {spec.name}, rows 0 and 7, all heads path={path}")
    inp = synth.scan_inputs(spec)
    y, fin = run_gpu(inp, spec.chunk)
    for b in (0, 7):
        row = {k: (v if k in ("A", "D") or v is None else v[b:b + 1]) for k, v in inp.items()}
        yo, fo = oracle.scan(**oracle_args(row))
        ey = rel_err(f64(y[b:b + 1]), yo)
        ef = rel_err(f64(fin[b:b + 1]), fo)
        print(f"  row {b}: rel_err y {ey:.3e} final {ef:.3e}", flush=True)
        assert ey <= TOL[torch.bfloat16], f"row {b} y rel err {ey:.3e}"
        assert ef <= TOL[torch.bfloat16], f"row {b} final rel err {ef:.3e}"
        del yo, fo


@pytest.mark.parametrize("path", ["auto", "separate"])
def test_offsets_past_2gib(path, monkeypatch):
    """x, y, B and C past 2^31 bytes: 4,194,381 tokens x 8 heads of headdim 64
    (4.3 GB of bf16 x, 16,385 chunks with a 77-token last one), inputs drawn
    on the device.  The oracle checks 333 tokens from two cut points, the
    chunk that starts at byte 2^31 of x and the last full chunk with the
    tail (and the final state), each from the state the GPU reaches at the
    cut (a prefix call).  The automatic choice chains the state pass."""
    if path == "separate":
        monkeypatch.setenv("SSD_PREFILL_PATH", "separate")
    Bt, L, H, P, N, G, Q = 1, (1 << 22) + 77, 8, 64, 128, 1, 256
    announce(f"scan_fwd {L} tokens x {H} heads, past 2 GiB, path={path}")
    gen = torch.Generator(device=DEV).manual_seed(61)
    bf = torch.bfloat16
    x = torch.randn((Bt, L, H, P), generator=gen, device=DEV, dtype=bf)
    B = torch.randn((Bt, L, G, N), generator=gen, device=DEV, dtype=bf)
    C = torch.randn((Bt, L, G, N), generator=gen, device=DEV, dtype=bf)
    dt = torch.rand((Bt, L, H), generator=gen, device=DEV) * 0.099 + 0.001
    A = -torch.exp(torch.rand((H,), generator=gen, device=DEV) * float(np.log(16.0)))
    D = torch.randn((H,), generator=gen, device=DEV)
    init = torch.randn((Bt, H, P, N), generator=gen, device=DEV) * 0.1
    assert x.numel() * x.element_size() > (1 << 32)
    ws = torch.empty(ssd.workspace_size(Bt, L, H, P, N, G, Q, bf), dtype=torch.uint8, device=DEV)
    y, fin = ssd.scan_fwd(x, dt, A, B, C, D, chunk=Q, init_state=init, workspace=ws)
    torch.cuda.synchronize()
    err = binding.error_word(ws, binding._scan_desc(x, B, Q))
    assert err in (None, 0), f"a hand-off wait ran out (error word {err})"
    del ws
    T = -(-L // Q)
    tol = TOL[bf]
    for L0 in ((T // 2) * Q, (T - 2) * Q):
        _, f0 = ssd.scan_fwd(x[:, :L0], dt[:, :L0], A, B[:, :L0], C[:, :L0], D, chunk=Q,
                             init_state=init)
        torch.cuda.synchronize()
        n = min(333, L - L0)
        sl = slice(L0, L0 + n)
        yo, fo = oracle.scan(x[:, sl].cpu(), dt[:, sl].cpu(), A.cpu(), B[:, sl].cpu(),
                             C[:, sl].cpu(), D.cpu(), f0.cpu())
        ey = rel_err(f64(y[:, sl]), yo)
        print(f"  tokens {L0}..{L0 + n}: rel_err y {ey:.3e}", flush=True)
        assert ey <= tol, f"y rel err {ey:.3e} from token {L0}"
        if L0 + n == L:
            ef = rel_err(f64(fin), fo)
            print(f"  final state rel_err {ef:.3e}", flush=True)
            assert ef <= tol, f"final rel err {ef:.3e}"
        del f0
    del x, B, C, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["auto", "chained"])
def test_two_streams_at_once(path, monkeypatch):
    """Two prefill calls on two streams at the same time, each with its own
    workspace, give bit for bit what each gives alone: the library keeps no
    per-call state outside the caller's buffers (the chained state pass's
    flags and error word included)."""
    if path == "chained":
        monkeypatch.setenv("SSD_PREFILL_PATH", "chained")
    specs = [synth.WORKLOADS["m130m_bf16"],
             synth.custom_spec(2, 1000, 16, 64, 128, 2, 256, "bf16", dt_rule="ranged",
                               init="normal", seed=81)]
    announce(f"two streams path={path}")
    runs = []
    for spec in specs:
        d = to_dev(synth.scan_inputs(spec), DEV)
        x = d["x"]
        ws = torch.empty(ssd.workspace_size(*x.shape, d["B"].shape[3], d["B"].shape[2],
                                            spec.chunk, x.dtype), dtype=torch.uint8, device=DEV)
        y0, f0 = ssd.scan_fwd(x, d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=spec.chunk,
                              init_state=d["init"], workspace=ws)
        runs.append((spec, d, ws, y0, f0))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    outs = []
    for rep in range(3):
        for (spec, d, ws, _, _), s in zip(runs, streams):
            with torch.cuda.stream(s):
                outs.append(ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                         chunk=spec.chunk, init_state=d["init"], workspace=ws))
    torch.cuda.synchronize()
    for i, (y, f) in enumerate(outs):
        spec, d, ws, y0, f0 = runs[i % len(runs)]
        assert torch.equal(y, y0) and torch.equal(f, f0), (i, spec.name)
        err = binding.error_word(ws, binding._scan_desc(d["x"], d["B"], spec.chunk))
        assert err in (None, 0)


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
    (1, 600, 4, 64, 128, 2, 256, "f32"),     # fp32 at chunk 256: three chunks, ragged
]


def mfma_shape(P, N, chunk, dt_):
    return dt_ == "bf16" and P == 64 and N in (64, 128) and chunk in (64, 128, 256)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("with_init", [True, False])
@pytest.mark.parametrize("path", ["auto", "chained"])
def test_shapes_full(shape, with_init, path, monkeypatch):
    Bt, L, H, P, N, G, chunk, dt_ = shape
    if path == "chained":
        if not mfma_shape(P, N, chunk, dt_):
            pytest.skip("the chained state pass runs on the MFMA shapes")
        monkeypatch.setenv("SSD_PREFILL_PATH", "chained")
    announce(f"scan_fwd shape {shape} init={with_init} path={path}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk, dt_, dt_rule="ranged",
                             init="normal" if with_init else "zero", seed=SHAPES.index(shape))
    inp = synth.scan_inputs(spec)
    check_full(inp, chunk, torch.bfloat16 if dt_ == "bf16" else torch.float32)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("path", ["separate", "chained"])
def test_chunk_sizes_agree_with_oracle(chunk, path, monkeypatch):
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    announce(f"chunk invariance chunk={chunk} path={path}")
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


@pytest.mark.parametrize("path", ["separate", "chained"])
def test_final_state_in_place(path, monkeypatch):
    """final_state may be init_state: every initial state is read before the
    final one overwrites it (on the chained path, by the chunk that ends the
    sequence, long after its first chunk read the initial state)."""
    monkeypatch.setenv("SSD_PREFILL_PATH", path)
    announce(f"final_state aliases init_state path={path}")
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
    (1, 600, 4, 64, 128, 2, 256, "f32"),     # fp32 at chunk 256, ragged
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


@pytest.mark.parametrize("grp", ["1", "2", "4", "8"])
def test_chain_groups(grp, monkeypatch):
    """Every hand-off grouping of the single-kernel path (chunks per group,
    forced through SSD_CHAIN_GROUP): several batch rows, a ragged last chunk,
    a chain longer than a group, and the final state written over the init
    state it started from."""
    monkeypatch.setenv("SSD_PREFILL_PATH", "fused")
    monkeypatch.setenv("SSD_CHAIN_GROUP", grp)
    spec = synth.custom_spec(2, 9 * 256 + 77, 6, 64, 128, 2, 256, "bf16", dt_rule="ranged",
                             init="normal", seed=21)
    announce(f"chain group {grp} {spec}")
    inp = synth.scan_inputs(spec)
    d = to_dev(inp, DEV)
    h = d["init"].clone()
    x = d["x"]
    ws = torch.empty(ssd.workspace_size(2, spec.seqlen, 6, 64, 128, 2, 256, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    y, fin = ssd.scan_fwd(x, d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=256, init_state=h,
                          final_state=h, workspace=ws)
    torch.cuda.synchronize()
    assert binding.error_word(ws, binding._scan_desc(x, d["B"], 256)) == 0
    yo, fo = oracle.scan(**oracle_args(inp))
    ey, ef = rel_err(f64(y), yo), rel_err(f64(h), fo)
    print(f"  rel_err y {ey:.3e} final {ef:.3e}", flush=True)
    assert ey <= TOL[torch.bfloat16] and ef <= TOL[torch.bfloat16]


FUSED_SHAPES = [
    # Bt, L, H, P, N, G: chunk 256, bf16 (the single-kernel path's scope)
    (2, 513, 4, 64, 128, 2),     # ragged last chunk, two groups
    (1, 100, 3, 64, 64, 1),      # one partial chunk
    (3, 1024, 8, 64, 128, 4),    # four full chunks, four groups
    (1, 2048, 24, 64, 128, 1),   # the 130M head shape
]


@pytest.mark.parametrize("queues", ["1", "8"])
@pytest.mark.parametrize("shape", FUSED_SHAPES)
def test_fused_path_shapes(shape, queues, monkeypatch):
    """The opt-in single-kernel prefill against the oracle, with one work
    queue and with one queue per XCD."""
    monkeypatch.setenv("SSD_PREFILL_PATH", "fused")
    monkeypatch.setenv("SSD_CHAIN_QUEUES", queues)
    Bt, L, H, P, N, G = shape
    announce(f"fused path {shape} queues {queues}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, 256, "bf16", dt_rule="ranged", init="normal",
                             seed=31 + FUSED_SHAPES.index(shape))
    check_full(synth.scan_inputs(spec), 256, torch.bfloat16)


def test_fused_path_2p7b_sampled(monkeypatch):
    monkeypatch.setenv("SSD_PREFILL_PATH", "fused")
    spec = synth.WORKLOADS["m2p7b_bf16"]
    announce(f"fused path {spec.name} sampled heads")
    sampled_check(synth.scan_inputs(spec), spec.chunk, [(0, 0), (0, 33), (0, 79)],
                  torch.bfloat16)
