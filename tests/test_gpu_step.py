"""GPU parity of the cached decode step (through the C ABI) against the oracle.

The decode workload: 2.7B head shape (80 heads, headdim 64, d_state 128), fp32
state from N(0, 0.1), one token of bf16 x/B/C per step, 4096 sequential steps,
every step's y and the final state compared with the oracle recurrence (all
heads at batch 1, sampled (batch, head) pairs at batch 64).
"""
import numpy as np
import pytest
import torch

import oracle
import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import synth

from helpers import TOL, f64, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("shape", [
    # Bt, H, P, N, G, dtype
    (1, 4, 16, 16, 1, torch.float32),
    (3, 8, 64, 128, 2, torch.bfloat16),
    (2, 6, 5, 4, 3, torch.float32),
    (2, 4, 64, 256, 4, torch.bfloat16),
    (1, 80, 64, 128, 1, torch.bfloat16),
])
def test_single_step(shape):
    Bt, H, P, N, G, dtype = shape
    print(f"[case] step {shape}", flush=True)
    g = torch.Generator().manual_seed(7)
    state = torch.randn(Bt, H, P, N, generator=g) * 0.1
    x = torch.randn(Bt, H, P, generator=g).to(dtype)
    dt = torch.rand(Bt, H, generator=g) * 0.1
    A = -torch.rand(H, generator=g) * 8
    B = torch.randn(Bt, G, N, generator=g).to(dtype)
    C = torch.randn(Bt, G, N, generator=g).to(dtype)
    D = torch.randn(H, generator=g)
    yo, so = oracle.step(state, x, dt, A, B, C, D)
    sd = state.to(DEV)
    y = ssd.step(sd, x.to(DEV), dt.to(DEV), A.to(DEV), B.to(DEV), C.to(DEV), D.to(DEV))
    torch.cuda.synchronize()
    assert rel_err(f64(y), yo) <= TOL[dtype]
    assert rel_err(f64(sd), so) <= TOL[dtype]


def test_step_state_past_2gib():
    """One step at batch 1024 with the 2.7B head shape: 2.7 GB of fp32 state,
    rows past byte 2^31 of it.  Sampled batch rows (the first, the one that
    starts past 2^31 bytes, the last) against the oracle step; the inputs are
    drawn on the device."""
    Bt, H, P, N, G = 1024, 80, 64, 128, 1
    print(f"[case] step batch {Bt}, state past 2 GiB", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(71)
    bf = torch.bfloat16
    sd = torch.randn((Bt, H, P, N), generator=gen, device=DEV) * 0.1
    assert sd.numel() * 4 > (1 << 31)
    x = torch.randn((Bt, H, P), generator=gen, device=DEV, dtype=bf)
    dt = torch.rand((Bt, H), generator=gen, device=DEV) * 0.1
    A = -torch.rand((H,), generator=gen, device=DEV) * 8
    B = torch.randn((Bt, G, N), generator=gen, device=DEV, dtype=bf)
    C = torch.randn((Bt, G, N), generator=gen, device=DEV, dtype=bf)
    D = torch.randn((H,), generator=gen, device=DEV)
    rows = [0, (1 << 31) // (H * P * N * 4) + 1, Bt - 1]
    before = {b: sd[b:b + 1].cpu() for b in rows}
    y = ssd.step(sd, x, dt, A, B, C, D)
    torch.cuda.synchronize()
    for b in rows:
        sl = slice(b, b + 1)
        yo, so = oracle.step(before[b], x[sl].cpu(), dt[sl].cpu(), A.cpu(), B[sl].cpu(),
                             C[sl].cpu(), D.cpu())
        assert rel_err(f64(y[sl]), yo) <= TOL[bf], b
        assert rel_err(f64(sd[sl]), so) <= TOL[bf], b
    del sd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_2p7b_b1", "decode_2p7b_b64"])
def test_decode_chain_4096(name):
    spec = synth.DECODE_WORKLOADS[name]
    print(f"[case] decode chain {name}", flush=True)
    stream = synth.DecodeStream(spec)
    pairs = [(b, h) for b in range(spec.batch) for h in range(spec.nheads)] \
        if spec.batch == 1 else [(0, 0), (17, 33), (40, 5), (63, 79)]
    R = spec.nheads // spec.ngroups
    state0 = stream.state.clone()
    sd = stream.state.to(DEV)
    A, D = stream.A.to(DEV), stream.D.to(DEV)
    ys = []
    rec = {p: {k: [] for k in ("x", "dt", "B", "C")} for p in pairs}
    for t in range(spec.steps):
        s = stream.next_step()
        y = ssd.step(sd, s["x"].to(DEV), s["dt"].to(DEV), A, s["B"].to(DEV), s["C"].to(DEV), D)
        ys.append(torch.stack([y[b, h] for b, h in pairs]).float().cpu())
        for b, h in pairs:
            r, g = rec[(b, h)], h // R
            r["x"].append(s["x"][b, h])
            r["dt"].append(s["dt"][b, h])
            r["B"].append(s["B"][b, g])
            r["C"].append(s["C"][b, g])
    torch.cuda.synchronize()
    yg = torch.stack(ys, dim=1).numpy()                 # [pairs, steps, P]
    # the oracle runs each sampled (b, h) chain as one recurrence over the steps
    yo, fo = [], []
    for b, h in pairs:
        r = rec[(b, h)]
        x = torch.stack(r["x"])[None, :, None, :]
        dt = torch.stack(r["dt"])[None, :, None]
        Bs = torch.stack(r["B"])[None, :, None, :]
        Cs = torch.stack(r["C"])[None, :, None, :]
        y1, f1 = oracle.scan(x, dt, stream.A[h:h + 1], Bs, Cs, stream.D[h:h + 1],
                             state0[b:b + 1, h:h + 1])
        yo.append(y1[0, :, 0, :])
        fo.append(f1[0, 0])
    ey = rel_err(yg, np.stack(yo))
    ef = rel_err(np.stack([f64(sd[b, h]) for b, h in pairs]), np.stack(fo))
    assert ey <= TOL[torch.bfloat16], f"y rel err {ey:.3e}"
    assert ef <= TOL[torch.bfloat16], f"state rel err {ef:.3e}"


def test_decode_chain_batch64_all_rows():
    """The batch-64 decode workload over a 256-step chain of single steps:
    every y of every step and the whole final state against the oracle run as
    one recurrence over the same 256 tokens."""
    spec = synth.DECODE_WORKLOADS["decode_2p7b_b64"]
    print("[case] decode chain batch 64, all rows, 256 steps", flush=True)
    stream = synth.DecodeStream(spec)
    state0 = stream.state.clone()
    sd = stream.state.to(DEV)
    A, D = stream.A.to(DEV), stream.D.to(DEV)
    steps, ys = [], []
    for t in range(256):
        s = stream.next_step()
        steps.append(s)
        ys.append(ssd.step(sd, s["x"].to(DEV), s["dt"].to(DEV), A, s["B"].to(DEV),
                           s["C"].to(DEV), D).cpu())
    torch.cuda.synchronize()
    x = torch.stack([s["x"] for s in steps], dim=1)
    dt = torch.stack([s["dt"] for s in steps], dim=1)
    B = torch.stack([s["B"] for s in steps], dim=1)
    C = torch.stack([s["C"] for s in steps], dim=1)
    yo, fo = oracle.scan(x, dt, stream.A, B, C, stream.D, state0)
    ey = rel_err(f64(torch.stack(ys, dim=1)), yo)
    ef = rel_err(f64(sd), fo)
    assert ey <= TOL[torch.bfloat16], f"y rel err {ey:.3e}"
    assert ef <= TOL[torch.bfloat16], f"state rel err {ef:.3e}"


def test_decode_steps_match_prefill_on_gpu():
    """Steps through the GPU decode path agree with the GPU prefill path."""
    print("[case] decode == prefill", flush=True)
    spec = synth.custom_spec(2, 300, 8, 64, 128, 2, 64, "bf16", dt_rule="ranged",
                             init="normal", seed=21)
    inp = synth.scan_inputs(spec)
    d = to_dev(inp, DEV)
    y, fin = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=64,
                          init_state=d["init"])
    state = d["init"].clone()
    ys = []
    for t in range(spec.seqlen):
        ys.append(ssd.step(state, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                           d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"]))
    torch.cuda.synchronize()
    yo, fo = oracle.scan(**oracle_args(inp))
    assert rel_err(f64(torch.stack(ys, 1)), yo) <= TOL[torch.bfloat16]
    assert rel_err(f64(state), fo) <= TOL[torch.bfloat16]
    assert rel_err(f64(torch.stack(ys, 1)), f64(y)) <= 2 * TOL[torch.bfloat16]


def _multi_inputs(Bt, T, H, P, N, G, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    state = torch.randn(Bt, H, P, N, generator=g) * 0.1
    x = torch.randn(Bt, T, H, P, generator=g).to(dtype)
    dt = torch.rand(Bt, T, H, generator=g) * 0.1
    A = -torch.rand(H, generator=g) * 8
    B = torch.randn(Bt, T, G, N, generator=g).to(dtype)
    C = torch.randn(Bt, T, G, N, generator=g).to(dtype)
    D = torch.randn(H, generator=g)
    return state, x, dt, A, B, C, D


@pytest.mark.parametrize("shape", [
    # Bt, T, H, P, N, G, dtype
    (1, 1, 4, 16, 16, 1, torch.float32),
    (2, 7, 6, 5, 4, 3, torch.float32),
    (3, 64, 8, 64, 128, 2, torch.bfloat16),
    (2, 16, 4, 64, 256, 4, torch.bfloat16),
    (1, 33, 80, 64, 128, 1, torch.bfloat16),
    (2, 20, 3, 64, 16, 1, torch.float32),     # 64 rows per block, ragged token group
    (2, 5, 2, 96, 32, 2, torch.float32),      # 32 rows per block, headdim 3 blocks
    (1, 3, 2, 12, 32, 1, torch.bfloat16),     # headdim not a multiple of a block's rows
    (64, 3, 80, 64, 128, 1, torch.bfloat16),  # the batch-64 decode shape: 10240 step blocks
])
def test_step_multi_equals_chained_steps(shape):
    """nsteps tokens in one launch: bit for bit the chained single steps, and
    within tolerance of the oracle recurrence from the same state."""
    Bt, T, H, P, N, G, dtype = shape
    print(f"[case] step_multi {shape}", flush=True)
    state, x, dt, A, B, C, D = _multi_inputs(Bt, T, H, P, N, G, dtype, seed=11 + T)
    dv = [t.to(DEV) for t in (x, dt, A, B, C, D)]
    xd, dtd, Ad, Bd, Cd, Dd = dv
    s_multi = state.to(DEV)
    y_multi = ssd.step_multi(s_multi, xd, dtd, Ad, Bd, Cd, Dd)
    s_chain = state.to(DEV)
    y_chain = torch.stack([
        ssd.step(s_chain, xd[:, t].clone(), dtd[:, t].clone(), Ad,
                 Bd[:, t].clone(), Cd[:, t].clone(), Dd) for t in range(T)], dim=1)
    torch.cuda.synchronize()
    assert torch.equal(y_multi, y_chain)
    assert torch.equal(s_multi, s_chain)
    yo, fo = oracle.scan(x, dt, A, B, C, D, state)
    assert rel_err(f64(y_multi), yo) <= TOL[dtype]
    assert rel_err(f64(s_multi), fo) <= TOL[dtype]


def test_step_multi_decode_workload_batch64():
    """The 2.7B decode shape at batch 64, 32 tokens per launch, all rows
    against the oracle."""
    print("[case] step_multi batch 64", flush=True)
    spec = synth.DECODE_WORKLOADS["decode_2p7b_b64"]
    stream = synth.DecodeStream(spec)
    steps = [stream.next_step() for _ in range(32)]
    x = torch.stack([s["x"] for s in steps], dim=1)
    dt = torch.stack([s["dt"] for s in steps], dim=1)
    B = torch.stack([s["B"] for s in steps], dim=1)
    C = torch.stack([s["C"] for s in steps], dim=1)
    state0 = stream.state.clone()
    sd = state0.to(DEV)
    y = ssd.step_multi(sd, x.to(DEV), dt.to(DEV), stream.A.to(DEV), B.to(DEV), C.to(DEV),
                       stream.D.to(DEV))
    torch.cuda.synchronize()
    yo, fo = oracle.scan(x, dt, stream.A, B, C, stream.D, state0)
    assert rel_err(f64(y), yo) <= TOL[torch.bfloat16]
    assert rel_err(f64(sd), fo) <= TOL[torch.bfloat16]


def test_graph_captured_decode_chain():
    """A chain of decode steps captured in one HIP graph (no host work between
    tokens) reproduces the eager chain bit for bit on every replay, with eager
    work on the stream between replays."""
    print("[case] graph-captured decode", flush=True)
    Bt, T, H, P, N, G = 2, 24, 8, 64, 128, 2
    state, x, dt, A, B, C, D = _multi_inputs(Bt, T, H, P, N, G, torch.bfloat16, seed=5)
    xd, dtd, Ad, Bd, Cd, Dd = (t.to(DEV) for t in (x, dt, A, B, C, D))
    steps = [(xd[:, t].contiguous(), dtd[:, t].contiguous(), Bd[:, t].contiguous(),
              Cd[:, t].contiguous()) for t in range(T)]
    s_ref = state.to(DEV)
    y_ref = torch.stack([ssd.step(s_ref, xs, ds, Ad, bs, cs, Dd) for xs, ds, bs, cs in steps], 1)
    s_g = state.to(DEV)
    ys = [torch.empty_like(y_ref[:, 0]) for _ in range(T)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, (xs, ds, bs, cs) in enumerate(steps):
            ssd.step(s_g, xs, ds, Ad, bs, cs, Dd, y=ys[t])
    for rep in range(3):
        s_g.copy_(state.to(DEV))
        for yt in ys:
            yt.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.stack(ys, 1), y_ref), f"replay {rep}"
        assert torch.equal(s_g, s_ref), f"replay {rep}"


def test_graph_captured_prefill():
    """ssd_scan_fwd (three launches on the MFMA path) captured in a HIP graph
    equals the eager call bit for bit on every replay."""
    print("[case] graph-captured prefill", flush=True)
    spec = synth.custom_spec(1, 1000, 16, 64, 128, 2, 256, "bf16", dt_rule="ranged",
                             init="normal", seed=31)
    d = to_dev(synth.scan_inputs(spec), DEV)
    Bt, L, H, P, N, G = 1, 1000, 16, 64, 128, 2
    y_ref, f_ref = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=256,
                                init_state=d["init"])
    ws = torch.empty(ssd.workspace_size(Bt, L, H, P, N, G, 256, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty_like(y_ref)
    fin = torch.empty_like(f_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=256,
                     init_state=d["init"], final_state=fin, workspace=ws, y=y)
    for rep in range(3):
        y.zero_()
        fin.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"
        assert torch.equal(fin, f_ref), f"replay {rep}"
