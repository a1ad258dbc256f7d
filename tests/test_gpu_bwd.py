"""GPU parity of the scan gradient (ssd_scan_bwd, through the C ABI) against
the fp64 adjoint recurrence of the oracle (itself pinned to finite
differences of the forward oracle).

Every output is compared element by element (dx, ddt, dB, dC, dinit) or
whole (dA, dD) with the dtype's bar in the rel_err metric; bf16 inputs give
fp32-accumulated gradients from the same bf16 values the oracle sees."""
import sys

import numpy as np
import pytest
import torch

import oracle
import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import synth

from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def inputs(spec, seed, with_D=True, with_init=True, with_dfinal=True):
    inp = synth.scan_inputs(spec, seed=seed)
    rng = np.random.default_rng(seed + 1)
    dt_ = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    inp["dy"] = torch.from_numpy(rng.standard_normal(inp["x"].shape, dtype=np.float32)).to(dt_)
    Bt, H, P, N = spec.batch, spec.nheads, spec.headdim, spec.dstate
    inp["dfinal"] = (torch.from_numpy(rng.standard_normal((Bt, H, P, N), dtype=np.float32))
                     if with_dfinal else None)
    if not with_D:
        inp["D"] = None
    if not with_init:
        inp["init"] = None
    return inp


def run(inp, chunk):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    g = ssd.scan_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["dy"], d["D"], d["init"],
                     d["dfinal"], chunk=chunk)
    torch.cuda.synchronize()
    return g


def reference(inp):
    return oracle.scan_vjp(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                           inp["init"], dy=inp["dy"], dfinal=inp["dfinal"])


def check(g, ref, tol, keys=GRADS):
    for k in keys:
        if g.get(k) is None:
            continue
        e = rel_err(f64(g[k]), ref[k])
        assert e <= tol, (k, e)


SHAPES = {
    # Bt, L, H, P, N, G, dtype
    "f32_ragged": (2, 100, 4, 16, 16, 2, "f32"),
    "f32_odd": (1, 33, 3, 5, 4, 1, "f32"),
    "bf16_2p7b_heads": (1, 300, 4, 64, 128, 1, "bf16"),
    "f32_max_slices": (1, 40, 2, 256, 256, 2, "f32"),
    "bf16_groups": (2, 70, 8, 32, 64, 4, "bf16"),
    # headdim 64, d_state 64 / 128 (the matrix-core kernel): 3 and 5 heads per
    # group (partial head slices), two groups, and a last chunk of one token
    "bf16_n64_groups": (2, 77, 6, 64, 64, 2, "bf16"),
    "bf16_n128_groups": (1, 45, 10, 64, 128, 2, "bf16"),
    "bf16_n64_one_token_tail": (1, 33, 4, 64, 64, 1, "bf16"),
    # enough 64-token chunks that the kernel takes several heads per block,
    # with a shorter last slice (11 heads: slices of 6 and 5 on 256 CUs)
    "bf16_heads_per_block": (4, 2048, 11, 64, 64, 1, "bf16"),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_bwd_vs_oracle(name):
    Bt, L, H, P, N, G, dt_ = SHAPES[name]
    announce(f"bwd {name}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=64, dtype=dt_, dt_rule="ranged",
                             init="normal", seed=11)
    inp = inputs(spec, seed=11)
    g = run(inp, 64)
    check(g, reference(inp), TOL[inp["x"].dtype])


@pytest.mark.parametrize("opt", ["no_D", "no_init", "no_dfinal", "none"])
def test_bwd_optional_inputs(opt):
    announce(f"bwd optional {opt}")
    spec = synth.custom_spec(1, 90, 4, 16, 32, 2, chunk=32, dtype="f32", dt_rule="ranged",
                             init="normal", seed=12)
    inp = inputs(spec, seed=12, with_D=opt not in ("no_D", "none"),
                 with_init=opt not in ("no_init", "none"),
                 with_dfinal=opt not in ("no_dfinal", "none"))
    g = run(inp, 32)
    ref = reference(inp)
    check(g, ref, TOL[torch.float32])
    assert (g["dD"] is None) == (inp["D"] is None)


def test_bwd_130m_full():
    """The 130M head shape (24 heads, headdim 64, d_state 128) at 2048 tokens,
    the pages' training-step comparison scale; every output checked."""
    announce("bwd 130M 2048")
    spec = synth.WORKLOADS["m130m_bf16"]
    inp = inputs(spec, seed=13)
    g = run(inp, spec.chunk)
    check(g, reference(inp), TOL[torch.bfloat16])


def test_bwd_2p7b_sampled_and_repeatable():
    """The 2.7B prefill workload (4096 tokens, 80 heads): per-head gradients of
    6 sampled heads against the oracle on that head alone (dB and dC sum over
    all heads, so they are checked at the 130M scale above); dx, ddt and dinit
    bit for bit equal over two runs."""
    announce("bwd 2.7B sampled")
    spec = synth.WORKLOADS["m2p7b_bf16"]
    inp = inputs(spec, seed=14)
    g = run(inp, spec.chunk)
    g2 = run(inp, spec.chunk)
    for k in ("dx", "ddt", "dinit"):
        assert torch.equal(g[k], g2[k]), k
    for h in (0, 17, 33, 48, 61, 79):
        sl = {k: inp[k] for k in ("B", "C")}
        ref = oracle.scan_vjp(inp["x"][:, :, h:h + 1], inp["dt"][:, :, h:h + 1],
                              inp["A"][h:h + 1], sl["B"], sl["C"], inp["D"][h:h + 1],
                              inp["init"][:, h:h + 1], dy=inp["dy"][:, :, h:h + 1],
                              dfinal=inp["dfinal"][:, h:h + 1])
        tol = TOL[torch.bfloat16]
        assert rel_err(f64(g["dx"][:, :, h]), ref["dx"][:, :, 0]) <= tol, h
        assert rel_err(f64(g["ddt"][:, :, h]), ref["ddt"][:, :, 0]) <= tol, h
        assert rel_err(f64(g["dinit"][:, h]), ref["dinit"][:, 0]) <= tol, h
        assert rel_err(np.array([float(g["dA"][h])]), ref["dA"]) <= tol, h
        assert rel_err(np.array([float(g["dD"][h])]), ref["dD"]) <= tol, h


def test_bwd_past_2gib():
    """The gradient of a 4,194,381-token x 8-head prefill (4.3 GB of bf16 x
    and dy, 65,537 gradient chunks), inputs drawn on the device.  The last
    333 tokens (byte offsets past 2^32) are checked: the oracle's VJP of that
    suffix, started from the forward state the GPU reaches at the cut (a
    prefix call), with the same dy and dfinal, gives their dx, ddt, dB and
    dC (dA, dD and dinit sum over the whole sequence)."""
    Bt, L, H, P, N, G, Q = 1, (1 << 22) + 77, 8, 64, 128, 1, 256
    announce(f"bwd {L} tokens x {H} heads, past 2 GiB")
    gen = torch.Generator(device=DEV).manual_seed(65)
    bf = torch.bfloat16
    x = torch.randn((Bt, L, H, P), generator=gen, device=DEV, dtype=bf)
    dy = torch.randn((Bt, L, H, P), generator=gen, device=DEV, dtype=bf)
    B = torch.randn((Bt, L, G, N), generator=gen, device=DEV, dtype=bf)
    C = torch.randn((Bt, L, G, N), generator=gen, device=DEV, dtype=bf)
    dt = torch.rand((Bt, L, H), generator=gen, device=DEV) * 0.099 + 0.001
    A = -torch.exp(torch.rand((H,), generator=gen, device=DEV) * float(np.log(16.0)))
    D = torch.randn((H,), generator=gen, device=DEV)
    init = torch.randn((Bt, H, P, N), generator=gen, device=DEV) * 0.1
    dfinal = torch.randn((Bt, H, P, N), generator=gen, device=DEV)
    g = ssd.scan_bwd(x, dt, A, B, C, dy, D, init, dfinal, chunk=Q)
    torch.cuda.synchronize()
    L0 = L - 333
    _, h0 = ssd.scan_fwd(x[:, :L0], dt[:, :L0], A, B[:, :L0], C[:, :L0], D, chunk=Q,
                         init_state=init)
    torch.cuda.synchronize()
    sl = slice(L0, L)
    ref = oracle.scan_vjp(x[:, sl].cpu(), dt[:, sl].cpu(), A.cpu(), B[:, sl].cpu(),
                          C[:, sl].cpu(), D.cpu(), h0.cpu(), dy=dy[:, sl].cpu(),
                          dfinal=dfinal.cpu())
    for k in ("dx", "ddt", "dB", "dC"):
        e = rel_err(f64(g[k][:, sl]), ref[k])
        print(f"  {k} rel_err {e:.3e}", flush=True)
        assert e <= TOL[bf], (k, e)
    del g, x, dy, B, C
    torch.cuda.empty_cache()


EDGE_SHAPES = {
    "bf16_mfma": (1, 300, 4, 64, 128, 1, "bf16"),
    "bf16_mfma_groups": (2, 77, 6, 64, 64, 2, "bf16"),
    "f32_generic": (2, 100, 4, 16, 16, 2, "f32"),
}
EDGE_LIMIT = (1e-3, 0.05)   # inside the synthetic dt's range: some values clamp


@pytest.mark.parametrize("which", ["all", "gate", "dt"])
@pytest.mark.parametrize("name", list(EDGE_SHAPES))
def test_bwd_edges_vs_oracle(name, which):
    """The gradient through the fused edges (ssd_scan_bwd_ex): raw-dt gradient,
    dt_bias and gate gradients and every plain gradient against the oracle's
    chain rule over the fp64 adjoint (itself pinned to finite differences)."""
    Bt, L, H, P, N, G, dt_ = EDGE_SHAPES[name]
    announce(f"bwd edges {name} {which}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=64, dtype=dt_, dt_rule="ranged",
                             init="normal", seed=61)
    inp = synth.scan_edge_inputs(spec)
    rng = np.random.default_rng(62)
    io = torch.bfloat16 if dt_ == "bf16" else torch.float32
    dy = torch.from_numpy(rng.standard_normal(inp["x"].shape, dtype=np.float32)).to(io)
    dfinal = torch.from_numpy(rng.standard_normal(inp["init"].shape, dtype=np.float32))
    use_dt = which in ("all", "dt")
    use_gate = which in ("all", "gate")
    kw = dict(dt_bias=inp["dt_bias"], dt_softplus=True, dt_limit=EDGE_LIMIT) if use_dt else {}
    dt_in = inp["dt_raw"] if use_dt else inp["dt"]
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    g = ssd.scan_bwd(d["x"], dt_in.to(DEV), d["A"], d["B"], d["C"], dy.to(DEV), d["D"],
                     d["init"], dfinal.to(DEV), chunk=64,
                     z=d["gate"] if use_gate else None,
                     **{k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in kw.items()})
    torch.cuda.synchronize()
    ref = oracle.scan_vjp_edges(inp["x"], dt_in, inp["A"], inp["B"], inp["C"], inp["D"],
                                inp["init"], dy=dy, dfinal=dfinal,
                                dt_bias=inp["dt_bias"] if use_dt else None,
                                dt_softplus=use_dt, dt_limit=EDGE_LIMIT if use_dt else None,
                                z=inp["gate"] if use_gate else None)
    keys = list(GRADS) + (["dz"] if use_gate else []) + (["ddt_bias"] if use_dt else [])
    tol = TOL[io]
    for k in keys:
        e = rel_err(f64(g[k]), ref[k])
        assert e <= tol, (k, e)
    if use_dt:
        # the clamp holds some values: their raw-dt gradient is exactly zero
        assert bool((g["ddt"] == 0).any())


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("name", ["bf16_mfma_groups", "f32_generic"])
def test_bwd_edges_norm_vs_oracle(name, gated):
    """The gradient through the gated RMSNorm as well (norm groups = the B/C
    groups): dnorm_weight, dz and every other gradient against the oracle."""
    Bt, L, H, P, N, G, dt_ = EDGE_SHAPES[name]
    announce(f"bwd edges norm {name} gated {gated}")
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=64, dtype=dt_, dt_rule="ranged",
                             init="normal", seed=63)
    inp = synth.scan_edge_inputs(spec)
    rng = np.random.default_rng(64)
    io = torch.bfloat16 if dt_ == "bf16" else torch.float32
    dy = torch.from_numpy(rng.standard_normal(inp["x"].shape, dtype=np.float32)).to(io)
    dfinal = torch.from_numpy(rng.standard_normal(inp["init"].shape, dtype=np.float32))
    w = torch.from_numpy(1.0 + 0.5 * rng.standard_normal(H * P)).float()
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    g = ssd.scan_bwd(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], dy.to(DEV), d["D"], d["init"],
                     dfinal.to(DEV), chunk=64, dt_bias=d["dt_bias"], dt_softplus=True,
                     dt_limit=EDGE_LIMIT, z=d["gate"] if gated else None,
                     norm_weight=w.to(DEV), norm_eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.scan_vjp_edges(inp["x"], inp["dt_raw"], inp["A"], inp["B"], inp["C"],
                                inp["D"], inp["init"], dy=dy, dfinal=dfinal,
                                dt_bias=inp["dt_bias"], dt_softplus=True, dt_limit=EDGE_LIMIT,
                                z=inp["gate"] if gated else None, norm_weight=w, norm_eps=1e-5,
                                norm_groups=G)
    keys = list(GRADS) + ["ddt_bias", "dnorm_weight"] + (["dz"] if gated else [])
    tol = TOL[io]
    for k in keys:
        e = rel_err(f64(g[k]), ref[k])
        assert e <= tol, (k, e)


def test_graph_captured_bwd_with_edges():
    """ssd_scan_bwd_ex with the dt activation and the gate, captured in a HIP
    graph (its zero fills are kernels, not memsets), replayed three times with
    eager work in between: the deterministic outputs (dx, ddt, dinit, dz,
    ddt_bias) equal the eager call bit for bit; the atomically accumulated
    ones (dA, dB, dC, dD) to fp32 summation-order level."""
    announce("bwd edges graph replay")
    Bt, L, H, P, N, G = 1, 1000, 16, 64, 128, 2
    spec = synth.custom_spec(Bt, L, H, P, N, G, chunk=256, dtype="bf16", dt_rule="ranged",
                             init="normal", seed=91)
    inp = synth.scan_edge_inputs(spec)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    rng = np.random.default_rng(92)
    dy = torch.from_numpy(rng.standard_normal(inp["x"].shape, dtype=np.float32)).to(
        torch.bfloat16).to(DEV)
    dfin = torch.from_numpy(rng.standard_normal(inp["init"].shape, dtype=np.float32)).to(DEV)
    kw = dict(chunk=256, dt_bias=d["dt_bias"], dt_softplus=True, dt_limit=(1e-3, 0.05),
              z=d["gate"])
    args = (d["x"], d["dt_raw"], d["A"], d["B"], d["C"], dy, d["D"], d["init"], dfin)
    ref = ssd.scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = ssd.scan_bwd(*args, **kw)
    for rep in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(float("nan"))
        g.replay()
        # the program's own eager work between replays
        ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=256,
                     init_state=d["init"])
        torch.cuda.synchronize()
        for k in ("dx", "ddt", "dinit", "dz", "ddt_bias"):
            assert torch.equal(out[k], ref[k]), (k, rep)
        for k in ("dA", "dB", "dC", "dD"):
            assert rel_err(f64(out[k]), f64(ref[k])) <= 1e-5, (k, rep)
