"""ssd_scan_fwd_noalloc (the prefill with the library's built-in scratch
instead of a caller workspace) against ssd_scan_fwd on the same inputs:
two calls in a row, the second smaller than the first, each through the C
ABI; results must be those of ssd_scan_fwd (same kernels, bit for bit), so
also within the parity bar."""
import ctypes
import sys

import pytest
import torch

import mamba_ssd_chunked_scan_amd as ssd
from mamba_ssd_chunked_scan_amd import binding, synth

from helpers import TOL, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def noalloc(d, chunk):
    x, B = d["x"], d["B"]
    y = torch.empty_like(x)
    fin = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32,
                      device=DEV)
    desc = binding._scan_desc(x, B, chunk)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = binding.lib().ssd_scan_fwd_noalloc(
        ctypes.byref(desc), P(x), P(d["dt"]), P(d["A"]), P(B), P(d["C"]), P(d["D"]),
        P(d["init"]), P(y), P(fin), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, binding.status_string(st)
    return y, fin


@pytest.mark.parametrize("path", ["auto", "chained"])
def test_noalloc_matches_scan_fwd_twice(path, monkeypatch):
    """Both state-pass arrangements: the chained one keeps its hand-off flags
    in the scratch too, cleared by a kernel on every call."""
    if path != "auto":
        monkeypatch.setenv("SSD_PREFILL_PATH", path)
    specs = [synth.WORKLOADS["m2p7b_bf16"],
             synth.custom_spec(2, 777, 8, 64, 128, 2, 256, "bf16", dt_rule="ranged",
                               init="normal", seed=51)]
    assert specs[1].batch * specs[1].seqlen * specs[1].nheads < \
        specs[0].batch * specs[0].seqlen * specs[0].nheads
    for spec in specs:
        print(f"[case] noalloc path={path} {spec}", flush=True)
        sys.stdout.flush()
        d = to_dev(synth.scan_inputs(spec), DEV)
        y0, f0 = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                              chunk=spec.chunk, init_state=d["init"])
        y1, f1 = noalloc(d, spec.chunk)
        torch.cuda.synchronize()
        assert rel_err(f64(y1), f64(y0)) <= TOL[torch.bfloat16]
        assert rel_err(f64(f1), f64(f0)) <= TOL[torch.bfloat16]
        assert torch.equal(y1, y0) and torch.equal(f1, f0)
