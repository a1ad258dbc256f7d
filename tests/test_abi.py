"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any HIP call.  Every call here is built to fail validation (or to be a
documented no-op), so nothing is ever launched."""
import ctypes
import os
import re

import pytest

from mamba_ssd_chunked_scan_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, SCRATCH = range(8)

# fake device addresses: never dereferenced, since validation fails first
P16 = 0x10000
P_MIS = 0x10008


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "ssd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    declared = header_functions()
    assert set(declared) == set(binding.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    assert L.ssd_abi_version() == 12
    for s in range(8):
        assert binding.status_string(s)
    assert binding.status_string(99) == "unknown status"


def desc(**kw):
    d = dict(batch=1, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=256,
             dtype=1, reserved=0)
    d.update(kw)
    return binding.ScanDesc(**d)


def sdesc(**kw):
    d = dict(batch=2, nheads=8, headdim=64, dstate=128, ngroups=2, dtype=1, reserved=0)
    d.update(kw)
    return binding.StepDesc(**d)


def wsize(L, d):
    n = ctypes.c_size_t(12345)
    st = L.ssd_scan_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def cb_size(L, d):
    n = ctypes.c_size_t(12345)
    st = L.ssd_chunk_scan_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def r256(v):
    return (v + 255) // 256 * 256


def test_chunk_scan_workspace_size(L):
    # bf16, headdim 64, dstate 64/128, chunk 64/128/256: the MFMA kernels keep,
    # per (batch, chunk, group), one 4 KB C.B tile per causal 32x32 tile pair
    # and the chunk's C rows as MFMA operands (chunk * dstate bf16)
    for chunk, ni in ((256, 8), (128, 4), (64, 2)):
        for dstate in (64, 128):
            st, n = cb_size(L, desc(chunk=chunk, dstate=dstate))
            T = -(-512 // chunk)
            per = (ni * (ni + 1) // 2) * 4096 + chunk * dstate * 2
            assert st == OK and n == r256(1 * T * 2 * per)
    # ragged last chunk counts as a chunk
    assert cb_size(L, desc(seqlen=300, chunk=128)) == (OK, 3 * 2 * (10 * 4096 + 128 * 128 * 2))
    # shapes the generic kernels run keep the lower triangle (chunk (chunk+1)/2
    # values) of the fp32 C.B matrix per (batch, chunk, group)
    assert cb_size(L, desc(dtype=0)) == (OK, 1 * 2 * 2 * (256 * 257 // 2) * 4)
    assert cb_size(L, desc(headdim=32)) == (OK, 1 * 2 * 2 * (256 * 257 // 2) * 4)
    assert cb_size(L, desc(chunk=32)) == (OK, 1 * 16 * 2 * (32 * 33 // 2) * 4)
    assert cb_size(L, desc(dstate=256)) == (OK, 1 * 2 * 2 * (256 * 257 // 2) * 4)
    assert cb_size(L, desc(seqlen=0)) == (OK, 0)
    assert cb_size(L, desc(batch=0)) == (OK, 0)
    assert L.ssd_chunk_scan_workspace_size(ctypes.byref(desc()), None) == NULL
    assert cb_size(L, desc(chunk=48))[0] == UNSUP


def test_workspace_size(L):
    # the single-kernel path (chunk 256, bf16, headdim 64, dstate 64/128): a
    # 256-byte control block, one 8-byte flag per 32x32 state tile of every
    # (chunk, head), the C.B tiles and fragments, one hand-off state per
    # (chunk, head); or, if larger, the staged path's workspace (Acs, chunk
    # states, C.B tiles, activated dt, and on MFMA shapes the chained state
    # pass's 256 control bytes and one 8-byte flag per (chunk, head, wave)),
    # which the same shapes can also run
    T = 2
    chain = lambda slots, H=8: r256(256 + slots * H * 4 * 8)
    for dstate in (64, 128):
        st, n = wsize(L, desc(dstate=dstate))
        tiles = 2 * dstate // 32
        cbn = cb_size(L, desc(dstate=dstate))[1]
        fused = 256 + r256(T * 8 * tiles * 8) + cbn + r256(T * 8 * 64 * dstate * 4)
        staged = (2 * r256(8 * 512 * 4) + r256(T * 8 * 64 * dstate * 4) + cbn) + chain(T)
        assert st == OK and n == max(fused, staged)
    # the staged path: Acs, chunk states, the chunk-output workspace, the
    # activated dt, the chain's flags
    acs = 1 * 8 * 512 * 4
    states = 1 * T * 8 * 64 * 128 * 4
    st, n = wsize(L, desc(chunk=128))
    T128 = 4
    assert st == OK and n == (r256(acs) + r256(T128 * 8 * 64 * 128 * 4)
                              + cb_size(L, desc(chunk=128))[1] + r256(acs) + chain(T128))
    # ragged last chunk counts as a chunk
    st, n = wsize(L, desc(seqlen=300, chunk=128))
    assert st == OK and n == (r256(8 * 300 * 4) + r256(3 * 8 * 64 * 128 * 4)
                              + cb_size(L, desc(seqlen=300, chunk=128))[1] + r256(8 * 300 * 4)
                              + chain(3))
    # the generic kernels (fp32) pass states in a launch of their own: no chain
    st, n = wsize(L, desc(dtype=0))
    assert st == OK and n == r256(acs) + r256(states) + cb_size(L, desc(dtype=0))[1] + r256(acs)
    assert wsize(L, desc(seqlen=0)) == (OK, 0)
    assert wsize(L, desc(batch=0)) == (OK, 0)
    assert L.ssd_scan_workspace_size(ctypes.byref(desc()), None) == NULL


def test_error_word_offset(L, monkeypatch):
    off = ctypes.c_size_t(99)
    # on small grids the stage kernels (the default) pass states in a launch
    # of their own: no hand-off wait
    monkeypatch.delenv("SSD_PREFILL_PATH", raising=False)
    assert L.ssd_scan_error_word(ctypes.byref(desc()), ctypes.byref(off)) == UNSUP
    # large grids chain the state pass through the chunk-state blocks (from
    # 4096 blocks on when no device is visible to count compute units)
    big = desc(batch=8, seqlen=16384, nheads=80, ngroups=8)
    assert L.ssd_scan_error_word(ctypes.byref(big), ctypes.byref(off)) == OK
    # forced, the chain keeps its error word in its control words, after Acs,
    # the chunk states, the C.B tiles and the activated dt
    monkeypatch.setenv("SSD_PREFILL_PATH", "chained")
    T = 2
    cbn = cb_size(L, desc())[1]
    assert L.ssd_scan_error_word(ctypes.byref(desc()), ctypes.byref(off)) == OK
    assert off.value == 2 * r256(8 * 512 * 4) + r256(T * 8 * 64 * 128 * 4) + cbn + 4
    st = L.ssd_scan_error_word(ctypes.byref(desc(chunk=128)), ctypes.byref(off))
    assert st == OK and off.value == (2 * r256(8 * 512 * 4) + r256(4 * 8 * 64 * 128 * 4)
                                      + cb_size(L, desc(chunk=128))[1] + 4)
    # the generic kernels have no hand-off wait, nor has the separate state pass
    for kw in (dict(dtype=0), dict(headdim=32), dict(seqlen=0)):
        assert L.ssd_scan_error_word(ctypes.byref(desc(**kw)), ctypes.byref(off)) == UNSUP
    monkeypatch.setenv("SSD_PREFILL_PATH", "separate")
    assert L.ssd_scan_error_word(ctypes.byref(desc()), ctypes.byref(off)) == UNSUP
    monkeypatch.setenv("SSD_PREFILL_PATH", "fused")
    # the single-kernel path keeps its error word at byte 4 of the workspace
    assert L.ssd_scan_error_word(ctypes.byref(desc()), ctypes.byref(off)) == OK and off.value == 4
    assert L.ssd_scan_error_word(ctypes.byref(desc(dstate=64)), ctypes.byref(off)) == OK
    # shapes the single kernel does not run: the stage kernels' path (here
    # small grids: the separate state pass), or the generic kernels
    for kw in (dict(chunk=128), dict(dtype=0), dict(headdim=32), dict(seqlen=0)):
        assert L.ssd_scan_error_word(ctypes.byref(desc(**kw)), ctypes.byref(off)) == UNSUP
    assert L.ssd_scan_error_word(ctypes.byref(desc(chunk=48)), ctypes.byref(off)) == UNSUP
    assert L.ssd_scan_error_word(ctypes.byref(desc(nheads=0)), ctypes.byref(off)) == SHAPE
    assert L.ssd_scan_error_word(ctypes.byref(desc()), None) == NULL
    assert L.ssd_scan_error_word(None, ctypes.byref(off)) == NULL
    vd = binding.VarlenDesc(3, 900, 8, 64, 128, 2, 256, 1, 0)
    assert L.ssd_varlen_error_word(ctypes.byref(vd), ctypes.byref(off)) == OK and off.value == 4
    vd = binding.VarlenDesc(3, 900, 8, 64, 128, 2, 64, 1, 0)
    assert L.ssd_varlen_error_word(ctypes.byref(vd), ctypes.byref(off)) == UNSUP
    monkeypatch.setenv("SSD_PREFILL_PATH", "chained")
    assert L.ssd_varlen_error_word(ctypes.byref(vd), ctypes.byref(off)) == OK
    vd = binding.VarlenDesc(3, 900, 8, 64, 128, 2, 64, 0, 0)
    assert L.ssd_varlen_error_word(ctypes.byref(vd), ctypes.byref(off)) == UNSUP


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), SHAPE), (dict(seqlen=-5), SHAPE), (dict(nheads=0), SHAPE),
    (dict(headdim=0), SHAPE), (dict(dstate=0), SHAPE), (dict(ngroups=0), SHAPE),
    (dict(nheads=6, ngroups=4), SHAPE),
    (dict(chunk=48), UNSUP), (dict(chunk=8), UNSUP), (dict(chunk=512), UNSUP),
    (dict(dstate=96), UNSUP), (dict(dstate=2), UNSUP), (dict(dstate=512), UNSUP),
    (dict(headdim=257), UNSUP), (dict(dtype=2), UNSUP), (dict(reserved=1), UNSUP),
])
def test_scan_shape_errors(L, kw, status):
    d = desc(**kw)
    assert wsize(L, d)[0] == status
    ws = 1 << 30
    st = L.ssd_scan_fwd(ctypes.byref(d), P16, P16, P16, P16, P16, P16, P16, P16, P16, P16, ws,
                        None)
    assert st == status
    assert L.ssd_chunk_cumsum(ctypes.byref(d), P16, P16, P16, None) == status
    assert L.ssd_chunk_state(ctypes.byref(d), P16, P16, P16, P16, P16, None) == status
    assert L.ssd_state_passing(ctypes.byref(d), P16, P16, P16, P16, None) == status
    assert L.ssd_chunk_scan(ctypes.byref(d), P16, P16, P16, P16, P16, P16, P16, P16, P16,
                            ws, None) == status


def test_null_desc(L):
    assert L.ssd_scan_fwd(None, *([P16] * 10), 0, None) == NULL
    assert L.ssd_step(None, *([P16] * 8), None) == NULL
    assert L.ssd_chunk_cumsum(None, P16, P16, P16, None) == NULL


@pytest.mark.parametrize("which", range(6))
def test_scan_null_required_pointer(L, which):
    ptrs = [P16] * 10   # x dt A B C D init y final ws
    req = [0, 1, 2, 3, 4, 7]
    ptrs[req[which]] = None
    st = L.ssd_scan_fwd(ctypes.byref(desc()), *ptrs, 1 << 30, None)
    assert st == NULL


@pytest.mark.parametrize("which", range(10))
def test_scan_misaligned_pointer(L, which):
    ptrs = [P16] * 10
    ptrs[which] = P_MIS
    st = L.ssd_scan_fwd(ctypes.byref(desc()), *ptrs, 1 << 30, None)
    assert st == ALIGN


def test_scan_workspace_too_small(L):
    d = desc()
    _, need = wsize(L, d)
    st = L.ssd_scan_fwd(ctypes.byref(d), *([P16] * 10), need - 1, None)
    assert st == WS
    ptrs = [P16] * 9 + [None]
    assert L.ssd_scan_fwd(ctypes.byref(d), *ptrs, need, None) == NULL


def test_chunk_cb_errors(L):
    d = desc()
    _, need = cb_size(L, d)
    assert L.ssd_chunk_cb(ctypes.byref(d), P16, P16, P16, need - 1, None) == WS
    assert L.ssd_chunk_cb(ctypes.byref(d), None, P16, P16, need, None) == NULL
    assert L.ssd_chunk_cb(ctypes.byref(d), P16, None, P16, need, None) == NULL
    assert L.ssd_chunk_cb(ctypes.byref(d), P16, P16, None, need, None) == NULL
    assert L.ssd_chunk_cb(ctypes.byref(d), P_MIS, P16, P16, need, None) == ALIGN
    assert L.ssd_chunk_cb(ctypes.byref(desc(chunk=48)), P16, P16, P16, need, None) == UNSUP
    # the generic kernels' C.B matrices are checked the same way
    g = desc(dtype=0)
    _, gneed = cb_size(L, g)
    assert gneed > 0
    assert L.ssd_chunk_cb(ctypes.byref(g), P16, P16, P16, gneed - 1, None) == WS
    assert L.ssd_chunk_cb(ctypes.byref(g), P16, P16, None, gneed, None) == NULL
    # shapes that need no workspace: a no-op, pointers untouched
    for kw in (dict(seqlen=0), dict(batch=0)):
        assert L.ssd_chunk_cb(ctypes.byref(desc(**kw)), None, None, None, 0, None) == OK


def test_chunk_scan_workspace_errors(L):
    d = desc()
    _, need = cb_size(L, d)
    assert need > 0
    args = [P16] * 8   # x dt B C D Acs states y
    assert L.ssd_chunk_scan(ctypes.byref(d), *args, P16, need - 1, None) == WS
    assert L.ssd_chunk_scan(ctypes.byref(d), *args, None, need, None) == NULL
    assert L.ssd_chunk_scan(ctypes.byref(d), *args, P_MIS, need, None) == ALIGN
    for which in (0, 1, 2, 3, 5, 6, 7):
        a = list(args)
        a[which] = None
        assert L.ssd_chunk_scan(ctypes.byref(d), *a, P16, need, None) == NULL


def test_step_multi_errors(L):
    d = sdesc()
    ptrs = [P16] * 9   # state x dt A B C D y
    assert L.ssd_step_multi(None, 4, *([P16] * 8), None) == NULL
    assert L.ssd_step_multi(ctypes.byref(d), -1, *([P16] * 8), None) == SHAPE
    for which in (0, 1, 2, 3, 4, 5, 7):
        a = [P16] * 8
        a[which] = None
        assert L.ssd_step_multi(ctypes.byref(d), 4, *a, None) == NULL
    for which in range(8):
        a = [P16] * 8
        a[which] = P_MIS
        assert L.ssd_step_multi(ctypes.byref(d), 4, *a, None) == ALIGN
    for kw, status in ((dict(nheads=6, ngroups=4), SHAPE), (dict(dstate=96), UNSUP),
                       (dict(dtype=3), UNSUP), (dict(reserved=2), UNSUP)):
        assert L.ssd_step_multi(ctypes.byref(sdesc(**kw)), 4, *([P16] * 8), None) == status
    # nothing to do: no pointer is touched
    assert L.ssd_step_multi(ctypes.byref(d), 0, *([None] * 8), None) == OK
    assert L.ssd_step_multi(ctypes.byref(sdesc(batch=0)), 4, *([None] * 8), None) == OK


def edges(**kw):
    e = dict(dt_bias=None, z=None, dt_min=0.0, dt_max=0.0, dt_softplus=0, dt_limit=0)
    e.update(kw)
    return binding.Edges(**e)


@pytest.mark.parametrize("kw,status", [
    (dict(dt_limit=1, dt_min=0.1, dt_max=0.01), UNSUP),       # empty clamp range
    (dict(dt_limit=1, dt_min=float("nan"), dt_max=1.0), UNSUP),
    (dict(z=P_MIS), ALIGN), (dict(dt_bias=P_MIS), ALIGN),
    # gated RMSNorm: eps below zero or NaN, groups that do not divide the
    # 8 heads, a misaligned weight
    (dict(norm_weight=P16, norm_eps=-1e-5), UNSUP),
    (dict(norm_weight=P16, norm_eps=float("nan")), UNSUP),
    (dict(norm_weight=P16, norm_eps=1e-5, norm_groups=3), SHAPE),
    (dict(norm_weight=P16, norm_eps=1e-5, norm_groups=-1), SHAPE),
    (dict(norm_weight=P_MIS, norm_eps=1e-5), ALIGN),
])
def test_edges_errors(L, kw, status):
    e = ctypes.byref(edges(**kw))
    d = desc()
    _, need = wsize(L, d)
    assert L.ssd_scan_fwd_ex(ctypes.byref(d), e, *([P16] * 10), need, None) == status
    assert L.ssd_step_ex(ctypes.byref(sdesc()), e, *([P16] * 8), None) == status
    assert L.ssd_step_multi_ex(ctypes.byref(sdesc()), e, 3, *([P16] * 8), None) == status


def test_edges_null_is_plain(L):
    """A NULL ssd_edges is the plain call: the same checks in the same order."""
    d = desc()
    _, need = wsize(L, d)
    for which in range(10):
        ptrs = [P16] * 10
        ptrs[which] = P_MIS
        assert L.ssd_scan_fwd_ex(ctypes.byref(d), None, *ptrs, need, None) == ALIGN
    assert L.ssd_scan_fwd_ex(ctypes.byref(d), None, *([P16] * 10), need - 1, None) == WS
    assert L.ssd_scan_fwd_ex(None, None, *([P16] * 10), need, None) == NULL
    assert L.ssd_step_ex(None, None, *([P16] * 8), None) == NULL
    assert L.ssd_step_multi_ex(ctypes.byref(sdesc()), None, -2, *([P16] * 8), None) == SHAPE
    # a valid clamp and softplus with an empty batch: nothing to do
    e = ctypes.byref(edges(dt_softplus=1, dt_limit=1, dt_min=1e-3, dt_max=0.1))
    assert L.ssd_scan_fwd_ex(ctypes.byref(desc(batch=0)), e, *([None] * 10), 0, None) == OK
    # without a weight the norm fields are not read
    e = ctypes.byref(edges(norm_eps=-1.0, norm_groups=3))
    assert L.ssd_scan_fwd_ex(ctypes.byref(desc(batch=0)), e, *([None] * 10), 0, None) == OK


def vdesc(**kw):
    d = dict(nseq=3, total=700, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=256,
             dtype=1, reserved=0)
    d.update(kw)
    return binding.VarlenDesc(**d)


def vwsize(L, d):
    n = ctypes.c_size_t(12345)
    st = L.ssd_varlen_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_varlen_workspace_size(L):
    # the workspace of one 700-token row with 700/256 + 3 = 5 chunk slots
    # (every sequence may end in a short chunk) on the single-kernel path
    # (control block, flags, C.B tiles, hand-off states), then the chunk
    # table (8 bytes a slot), the sequence table (8 bytes a sequence) and the
    # slot positions (8 bytes a slot)
    slots = 700 // 256 + 3
    cbw = slots * 2 * (36 * 4096 + 256 * 128 * 2)
    st, n = vwsize(L, vdesc())
    assert st == OK
    fused = 256 + r256(slots * 8 * 8 * 8) + r256(cbw) + r256(slots * 8 * 64 * 128 * 4)
    staged = (2 * r256(8 * 700 * 4) + r256(slots * 8 * 64 * 128 * 4) + r256(cbw)
              + r256(256 + slots * 8 * 4 * 8))
    assert n == max(fused, staged) + 2 * r256(slots * 8) + r256(3 * 8)
    # the staged path (chunk 128): Acs, chunk states, C.B, activated dt
    slots = 700 // 128 + 3
    acs = 8 * 700 * 4
    states = slots * 8 * 64 * 128 * 4
    cbw = slots * 2 * (10 * 4096 + 128 * 128 * 2)
    st, n = vwsize(L, vdesc(chunk=128))
    assert st == OK
    assert n == (r256(acs) + r256(states) + r256(cbw) + r256(acs)
                 + r256(256 + slots * 8 * 4 * 8) + 2 * r256(slots * 8) + r256(3 * 8))
    assert vwsize(L, vdesc(nseq=0)) == (OK, 0)
    assert vwsize(L, vdesc(total=0)) == (OK, 0)
    assert L.ssd_varlen_workspace_size(ctypes.byref(vdesc()), None) == NULL


@pytest.mark.parametrize("kw,status", [
    (dict(nseq=-1), SHAPE), (dict(total=-3), SHAPE), (dict(nheads=6, ngroups=4), SHAPE),
    (dict(chunk=48), UNSUP), (dict(dstate=96), UNSUP), (dict(dtype=7), UNSUP),
    (dict(reserved=1), UNSUP), (dict(total=1 << 31), UNSUP), (dict(nseq=1 << 31), UNSUP),
])
def test_varlen_shape_errors(L, kw, status):
    d = vdesc(**kw)
    assert vwsize(L, d)[0] == status
    assert L.ssd_scan_fwd_varlen(ctypes.byref(d), None, *([P16] * 11), 1 << 30, None) == status


def test_varlen_pointer_errors(L):
    d = vdesc()
    _, need = vwsize(L, d)
    args = [P16] * 11   # cu x dt A B C D init y final ws
    assert L.ssd_scan_fwd_varlen(None, None, *args, need, None) == NULL
    for which in (0, 1, 2, 3, 4, 5, 8):   # required
        a = list(args)
        a[which] = None
        assert L.ssd_scan_fwd_varlen(ctypes.byref(d), None, *a, need, None) == NULL
    for which in range(11):
        a = list(args)
        a[which] = P_MIS
        assert L.ssd_scan_fwd_varlen(ctypes.byref(d), None, *a, need, None) == ALIGN
    assert L.ssd_scan_fwd_varlen(ctypes.byref(d), None, *args, need - 1, None) == WS
    a = list(args)
    a[10] = None
    assert L.ssd_scan_fwd_varlen(ctypes.byref(d), None, *a, need, None) == NULL
    e = ctypes.byref(edges(dt_limit=1, dt_min=1.0, dt_max=0.5))
    assert L.ssd_scan_fwd_varlen(ctypes.byref(d), e, *args, need, None) == UNSUP
    # no sequences: nothing is touched
    assert L.ssd_scan_fwd_varlen(ctypes.byref(vdesc(nseq=0)), None, *([None] * 11), 0,
                                 None) == OK
    # no tokens: only the state pointers are checked
    a = [None] * 11
    a[7] = P_MIS
    assert L.ssd_scan_fwd_varlen(ctypes.byref(vdesc(total=0)), None, *a, 0, None) == ALIGN


def test_bwd_workspace_and_errors(L):
    d = desc()   # batch 1, seqlen 512, 8 heads, headdim 64, dstate 128, bf16
    n = ctypes.c_size_t(0)
    assert L.ssd_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    # Acs, then the entering states and the end-state derivatives at the
    # gradient's own chunking: 64 tokens on the matrix-core path ...
    T64 = 512 // 64
    assert n.value == r256(8 * 512 * 4) + 2 * r256(T64 * 8 * 64 * 128 * 4)
    need = n.value
    # ... and 32 elsewhere (fp32 inputs; headdim 32)
    for other in (desc(dtype=0), desc(headdim=32)):
        assert L.ssd_scan_bwd_workspace_size(ctypes.byref(other), ctypes.byref(n)) == OK
        assert n.value == r256(8 * 512 * 4) + 2 * r256(16 * 8 * other.headdim * 128 * 4)
    args = [P16] * 16  # x dt A B C D init dy dfinal dx ddt dA dB dC dD dinit
    assert L.ssd_scan_bwd(None, *args, P16, need, None) == NULL
    for which in (0, 1, 2, 3, 4, 7, 9, 10, 11, 12, 13):   # required
        a = list(args)
        a[which] = None
        assert L.ssd_scan_bwd(ctypes.byref(d), *a, P16, need, None) == NULL, which
    for which in range(16):
        a = list(args)
        a[which] = P_MIS
        assert L.ssd_scan_bwd(ctypes.byref(d), *a, P16, need, None) == ALIGN, which
    assert L.ssd_scan_bwd(ctypes.byref(d), *args, P16, need - 1, None) == WS
    assert L.ssd_scan_bwd(ctypes.byref(d), *args, None, need, None) == NULL
    assert L.ssd_scan_bwd(ctypes.byref(desc(chunk=48)), *args, P16, need, None) == UNSUP
    assert L.ssd_scan_bwd(ctypes.byref(desc(nheads=6, ngroups=4)), *args, P16, need,
                          None) == SHAPE
    # a grid beyond 2^31 blocks at 32-token tiles, though fine for the forward's chunk
    big = desc(batch=1 << 22, seqlen=1 << 12, nheads=8, chunk=256)
    assert wsize(L, big)[0] == OK
    assert L.ssd_scan_bwd_workspace_size(ctypes.byref(big), ctypes.byref(n)) == UNSUP
    # no tokens: only dA (required) and the optional state pointers are checked
    a = [None] * 16
    assert L.ssd_scan_bwd(ctypes.byref(desc(seqlen=0)), *a, None, 0, None) == NULL
    a[11] = P_MIS
    assert L.ssd_scan_bwd(ctypes.byref(desc(seqlen=0)), *a, None, 0, None) == ALIGN


def test_empty_batch_is_noop(L):
    d = desc(batch=0)
    # all pointers NULL: nothing is touched and nothing is launched
    assert L.ssd_scan_fwd(ctypes.byref(d), *([None] * 10), 0, None) == OK
    assert L.ssd_chunk_cumsum(ctypes.byref(d), None, None, None, None) == OK
    s = sdesc(batch=0)
    assert L.ssd_step(ctypes.byref(s), *([None] * 8), None) == OK


def test_empty_sequence_checks_alignment(L):
    d = desc(seqlen=0)
    st = L.ssd_scan_fwd(ctypes.byref(d), *([None] * 6), P_MIS, None, P16, None, 0, None)
    assert st == ALIGN


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), SHAPE), (dict(nheads=0), SHAPE), (dict(nheads=6, ngroups=4), SHAPE),
    (dict(dstate=3), UNSUP), (dict(dstate=100), UNSUP), (dict(headdim=300), UNSUP),
    (dict(dtype=5), UNSUP), (dict(reserved=3), UNSUP),
])
def test_step_shape_errors(L, kw, status):
    assert L.ssd_step(ctypes.byref(sdesc(**kw)), *([P16] * 8), None) == status


@pytest.mark.parametrize("which", range(8))
def test_step_pointer_errors(L, which):
    ptrs = [P16] * 8   # state x dt A B C D y
    ptrs[which] = P_MIS
    assert L.ssd_step(ctypes.byref(sdesc()), *ptrs, None) == ALIGN
    if which != 6:   # D is optional
        ptrs[which] = None
        assert L.ssd_step(ctypes.byref(sdesc()), *ptrs, None) == NULL


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libssd.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()


def test_bwd_ex_workspace_and_errors(L):
    """ssd_scan_bwd_ex: NULL edges is ssd_scan_bwd (same workspace); a dt
    activation adds the activated dt; a gate adds the ungated output, the
    gated dy and the chunk-output stage's workspace; the norm's gradient is
    not built; a gate needs dz; dz and ddt_bias are alignment-checked."""
    d = desc()   # batch 1, seqlen 512, 8 heads, headdim 64, dstate 128, bf16
    n0, n1, n2 = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.ssd_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n0)) == OK
    assert L.ssd_scan_bwd_ex_workspace_size(ctypes.byref(d), None, ctypes.byref(n1)) == OK
    assert n0.value == n1.value
    ea = edges(dt_bias=P16, dt_softplus=1)
    assert L.ssd_scan_bwd_ex_workspace_size(ctypes.byref(d), ctypes.byref(ea),
                                            ctypes.byref(n1)) == OK
    parts = r256(8 * 1 * 4)                       # 8 heads x one 4096-row part
    assert n1.value == n0.value + r256(512 * 8 * 4) + parts
    eg = edges(dt_bias=P16, dt_softplus=1, z=P16)
    assert L.ssd_scan_bwd_ex_workspace_size(ctypes.byref(d), ctypes.byref(eg),
                                            ctypes.byref(n2)) == OK
    assert n2.value > n1.value + 2 * r256(512 * 8 * 64 * 2)
    # the norm's gradient: within the kernel's tiling it adds its partial sums;
    # headdim 12 (not a multiple of 8) is refused
    en = edges(dt_bias=P16, dt_softplus=1, z=P16, norm_weight=P16, norm_eps=1e-5)
    n3 = ctypes.c_size_t(0)
    assert L.ssd_scan_bwd_ex_workspace_size(ctypes.byref(d), ctypes.byref(en),
                                            ctypes.byref(n3)) == OK
    # 512 tokens x 2 groups over ~2048 blocks: one token per block, so 512
    # ranges of partial sums over the 512 channels, plus 512 / 64 rows of
    # their first-level sums
    assert n3.value == n2.value + r256((512 + 8) * 8 * 64 * 4)
    assert L.ssd_scan_bwd_ex_workspace_size(ctypes.byref(desc(headdim=12, dtype=0)),
                                            ctypes.byref(en), ctypes.byref(n1)) == UNSUP
    need = n3.value
    args = [P16] * 16  # x dt A B C D init dy dfinal dx ddt dA dB dC dD dinit
    assert L.ssd_scan_bwd_ex(ctypes.byref(d), ctypes.byref(eg), *args, None, P16, P16, P16, need,
                             None) == NULL                      # gate without dz
    assert L.ssd_scan_bwd_ex(ctypes.byref(d), ctypes.byref(eg), *args, P_MIS, P16, P16, P16, need,
                             None) == ALIGN
    assert L.ssd_scan_bwd_ex(ctypes.byref(d), ctypes.byref(eg), *args, P16, P_MIS, P16, P16, need,
                             None) == ALIGN
    assert L.ssd_scan_bwd_ex(ctypes.byref(d), ctypes.byref(en), *args, P16, P16, P_MIS, P16, need,
                             None) == ALIGN
    assert L.ssd_scan_bwd_ex(ctypes.byref(d), ctypes.byref(en), *args, P16, P16, P16, P16, need - 1,
                             None) == WS


def test_bwd_varlen_workspace_and_errors(L):
    """ssd_scan_bwd_varlen: the gradient's core at 64-token slots (total / 64
    + nseq of them) plus the chunk, sequence and slot tables; nothing for an empty
    batch; the same edge and pointer checks as ssd_scan_bwd_ex."""
    d = vdesc()   # 3 sequences, 700 tokens, 8 heads, headdim 64, dstate 128, bf16
    n = ctypes.c_size_t(0)
    assert L.ssd_scan_bwd_varlen_workspace_size(ctypes.byref(d), None, ctypes.byref(n)) == OK
    slots = 700 // 64 + 3
    core = r256(8 * 700 * 4) + 2 * r256(slots * 8 * 64 * 128 * 4)
    assert n.value == core + 2 * r256(slots * 8) + r256(3 * 8)
    assert L.ssd_scan_bwd_varlen_workspace_size(ctypes.byref(vdesc(nseq=0, total=0)), None,
                                                ctypes.byref(n)) == OK and n.value == 0
    eg = edges(dt_bias=P16, dt_softplus=1, z=P16)
    assert L.ssd_scan_bwd_varlen_workspace_size(ctypes.byref(d), ctypes.byref(eg),
                                                ctypes.byref(n)) == OK
    need = n.value
    args = [P16] * 17  # cu x dt A B C D init dy dfinal dx ddt dA dB dC dD dinit
    assert L.ssd_scan_bwd_varlen(ctypes.byref(d), ctypes.byref(eg), *args, None, P16, P16, P16,
                                 need, None) == NULL                # gate without dz
    for which in range(17):
        a = list(args)
        a[which] = P_MIS
        assert L.ssd_scan_bwd_varlen(ctypes.byref(d), ctypes.byref(eg), *a, P16, P16, P16, P16,
                                     need, None) == ALIGN, which
    assert L.ssd_scan_bwd_varlen(ctypes.byref(d), ctypes.byref(eg), *args, P16, P16, P16, P16,
                                 need - 1, None) == WS


def test_noalloc_checks(L):
    """ssd_scan_fwd_noalloc: every argument check runs before its first HIP
    call, and a shape whose workspace exceeds the built-in scratch is refused
    with SSD_ERR_SCRATCH (all of this without a device)."""
    ptrs = [P16] * 9  # x dt A B C D init y final
    assert L.ssd_scan_fwd_noalloc(None, *ptrs, None) == NULL
    assert L.ssd_scan_fwd_noalloc(ctypes.byref(desc(nheads=6, ngroups=4)), *ptrs, None) == SHAPE
    assert L.ssd_scan_fwd_noalloc(ctypes.byref(desc(chunk=48)), *ptrs, None) == UNSUP
    for which in (0, 1, 2, 3, 4, 7):   # the required pointers
        p = list(ptrs)
        p[which] = None
        assert L.ssd_scan_fwd_noalloc(ctypes.byref(desc()), *p, None) == NULL
    for which in range(9):
        p = list(ptrs)
        p[which] = P_MIS
        assert L.ssd_scan_fwd_noalloc(ctypes.byref(desc()), *p, None) == ALIGN
    # the batched long prefill (8 x 16384 tokens, 80 heads) needs ~2.3 GB
    big = desc(batch=8, seqlen=16384, nheads=80, ngroups=8)
    assert wsize(L, big)[1] > binding.NOALLOC_SCRATCH_BYTES
    assert L.ssd_scan_fwd_noalloc(ctypes.byref(big), *ptrs, None) == SCRATCH
    # the 2.7B head shape at 4096 tokens fits
    assert wsize(L, desc(seqlen=4096, nheads=80, ngroups=1))[1] <= binding.NOALLOC_SCRATCH_BYTES
    assert L.ssd_scan_fwd_noalloc(ctypes.byref(desc(batch=0)), *ptrs, None) == OK
    assert binding.status_string(SCRATCH).startswith("the call needs more device scratch")
