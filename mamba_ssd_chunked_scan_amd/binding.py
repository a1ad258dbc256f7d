"""ctypes binding of libssd (include/ssd.h).

Argument marshalling only: shapes and dtypes are checked, output tensors are
allocated with torch on the inputs' device, and the C entry point of the same
name runs the work on torch's current HIP stream.  There is no CPU or PyTorch
fallback: if libssd.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# SSD_LIB names another build of the library to load instead (the sanitizer
# test runs the argument checks against a host-sanitized build this way)
LIB_PATH = os.environ.get("SSD_LIB") or os.path.join(HERE, "libssd.so")

SSD_OK = 0
SSD_F32, SSD_BF16 = 0, 1
_STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL_PTR", 2: "SSD_ERR_SHAPE",
                 3: "SSD_ERR_UNSUPPORTED", 4: "SSD_ERR_ALIGN", 5: "SSD_ERR_WORKSPACE",
                 6: "SSD_ERR_HIP", 7: "SSD_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # include/ssd.h SSD_NOALLOC_SCRATCH_BYTES

# Every function include/ssd.h declares.
EXPORTS = ("ssd_status_string", "ssd_abi_version", "ssd_scan_workspace_size", "ssd_scan_fwd",
           "ssd_step", "ssd_step_multi", "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing",
           "ssd_chunk_scan_workspace_size", "ssd_chunk_cb", "ssd_chunk_scan", "ssd_scan_fwd_ex",
           "ssd_step_ex", "ssd_step_multi_ex", "ssd_varlen_workspace_size", "ssd_scan_fwd_varlen",
           "ssd_scan_bwd_workspace_size", "ssd_scan_bwd", "ssd_scan_bwd_ex_workspace_size",
           "ssd_scan_bwd_ex", "ssd_scan_bwd_varlen_workspace_size", "ssd_scan_bwd_varlen",
           "ssd_scan_error_word", "ssd_varlen_error_word", "ssd_scan_fwd_noalloc")


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class VarlenDesc(ctypes.Structure):
    _fields_ = [("nseq", ctypes.c_int64), ("total", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class StepDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Edges(ctypes.Structure):
    """ssd_edges: the dt activation and output gate fused into the scan, and
    the gated RMSNorm pass over its output."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
                ("dt_softplus", ctypes.c_int32), ("dt_limit", ctypes.c_int32),
                ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("norm_groups", ctypes.c_int32)]


class SSDError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} returned {_STATUS_NAMES.get(status, status)}: {text}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
ABI_VERSION = 12  # include/ssd.h: the structs above must match the library's


def lib() -> ctypes.CDLL:
    """The loaded libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mamba_ssd_chunked_scan_amd.build`"
                " (or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        L.ssd_status_string.argtypes = [ctypes.c_int]
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_abi_version.argtypes = []
        L.ssd_abi_version.restype = ctypes.c_int
        if L.ssd_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI {L.ssd_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild the library")
        L.ssd_scan_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                              ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_fwd.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 10 + [ctypes.c_size_t, _P]
        L.ssd_step.argtypes = [ctypes.POINTER(StepDesc)] + [_P] * 9
        L.ssd_step_multi.argtypes = [ctypes.POINTER(StepDesc), ctypes.c_int64] + [_P] * 9
        L.ssd_chunk_cumsum.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 4
        L.ssd_chunk_state.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 6
        L.ssd_state_passing.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 5
        L.ssd_chunk_scan_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_chunk_cb.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 3 + [ctypes.c_size_t, _P]
        L.ssd_chunk_scan.argtypes = ([ctypes.POINTER(ScanDesc)] + [_P] * 9
                                     + [ctypes.c_size_t, _P])
        L.ssd_scan_fwd_ex.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(Edges)]
                                      + [_P] * 10 + [ctypes.c_size_t, _P])
        L.ssd_step_ex.argtypes = [ctypes.POINTER(StepDesc), ctypes.POINTER(Edges)] + [_P] * 9
        L.ssd_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_bwd.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 17 + [ctypes.c_size_t, _P]
        L.ssd_scan_bwd_ex_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                                     ctypes.POINTER(Edges),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_bwd_ex.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(Edges)]
                                      + [_P] * 20 + [ctypes.c_size_t, _P])
        L.ssd_scan_bwd_varlen_workspace_size.argtypes = [ctypes.POINTER(VarlenDesc),
                                                         ctypes.POINTER(Edges),
                                                         ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_bwd_varlen.argtypes = ([ctypes.POINTER(VarlenDesc), ctypes.POINTER(Edges)]
                                          + [_P] * 21 + [ctypes.c_size_t, _P])
        L.ssd_varlen_workspace_size.argtypes = [ctypes.POINTER(VarlenDesc),
                                                ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_fwd_varlen.argtypes = ([ctypes.POINTER(VarlenDesc), ctypes.POINTER(Edges)]
                                          + [_P] * 11 + [ctypes.c_size_t, _P])
        L.ssd_step_multi_ex.argtypes = ([ctypes.POINTER(StepDesc), ctypes.POINTER(Edges),
                                         ctypes.c_int64] + [_P] * 9)
        L.ssd_scan_error_word.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanDesc)] + [_P] * 10
        L.ssd_varlen_error_word.argtypes = [ctypes.POINTER(VarlenDesc),
                                            ctypes.POINTER(ctypes.c_size_t)]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


def _check(fn, status):
    if status != SSD_OK:
        raise SSDError(fn, status, status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _io_dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise ValueError(f"x/B/C must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scan_desc(x, B, chunk):
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return ScanDesc(Bt, L, H, P, N, G, chunk, _io_dtype(x), 0)


def _check_scan_inputs(x, dt, A, B, C, D):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim], B [batch, seqlen, ngroups, dstate]")
    if x.device.type != "cuda":
        raise ValueError("inputs must be device tensors")
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, io = x.device, x.dtype
    _need(x, "x", (Bt, L, H, P), io, dev)
    _need(dt, "dt", (Bt, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (Bt, L, G, N), io, dev)
    if C is not None:
        _need(C, "C", (Bt, L, G, N), io, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    return Bt, L, H, P, N, G


def workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype) -> int:
    d = ScanDesc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                 SSD_BF16 if dtype == torch.bfloat16 else SSD_F32, 0)
    n = ctypes.c_size_t(0)
    _check("ssd_scan_workspace_size", lib().ssd_scan_workspace_size(ctypes.byref(d),
                                                                    ctypes.byref(n)))
    return n.value


def error_word(workspace, desc, varlen: bool = False):
    """The error word of a finished ssd_scan_fwd(_ex) / ssd_scan_fwd_varlen call
    that used ``workspace`` (a uint8 device tensor) for shape ``desc`` (a
    ScanDesc or VarlenDesc): 0 when every hand-off wait of the call completed,
    None when that shape runs no hand-off.  Reads device memory (synchronises
    with the workspace's device)."""
    off = ctypes.c_size_t(0)
    fn = lib().ssd_varlen_error_word if varlen else lib().ssd_scan_error_word
    st = fn(ctypes.byref(desc), ctypes.byref(off))
    if st == 3:  # SSD_ERR_UNSUPPORTED: no hand-off on this shape's path
        return None
    _check("ssd_varlen_error_word" if varlen else "ssd_scan_error_word", st)
    return int(workspace[off.value:off.value + 4].cpu().view(torch.int32).item())


def _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight=None, norm_eps=1e-5,
           norm_groups=0):
    """An Edges struct for the fused dt activation / output gate and the
    gated RMSNorm, or None when none is requested (the plain operation)."""
    if (dt_bias is None and not dt_softplus and dt_limit is None and z is None
            and norm_weight is None):
        return None
    e = Edges()
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", (H * P,), torch.float32, x.device)
        e.norm_weight = norm_weight.data_ptr()
        e.norm_eps = float(norm_eps)
        e.norm_groups = int(norm_groups)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", (H,), torch.float32, x.device)
        e.dt_bias = dt_bias.data_ptr()
    if z is not None:
        _need(z, "z", x.shape, x.dtype, x.device)
        e.z = z.data_ptr()
    e.dt_softplus = 1 if dt_softplus else 0
    if dt_limit is not None:
        lo, hi = dt_limit
        e.dt_min, e.dt_max, e.dt_limit = float(lo), float(hi), 1
    return e


def _eref(e):
    return None if e is None else ctypes.byref(e)


def scan_fwd(x, dt, A, B, C, D=None, chunk: int = 256, init_state=None,
             return_final_state: bool = True, final_state=None, workspace=None, y=None,
             dt_bias=None, dt_softplus: bool = False, dt_limit=None, z=None,
             norm_weight=None, norm_eps: float = 1e-5, norm_groups: int = 0):
    """Chunked SSD scan.  Returns (y, final_state); final_state is None when not requested.

    ``final_state`` may be a preallocated [batch, nheads, headdim, dstate] fp32
    tensor (it may be ``init_state`` itself); ``workspace`` a uint8 device tensor
    of at least :func:`workspace_size` bytes; ``y`` a preallocated output.
    Fused edges: ``dt_bias`` [nheads] fp32 is added to dt, ``dt_softplus``
    applies softplus, ``dt_limit`` = (lo, hi) clamps the result; ``z`` (x's
    shape and dtype) gates the output, y * silu(z).  ``norm_weight``
    [nheads * headdim] fp32 then applies the gated RMSNorm over
    ``norm_groups`` groups of whole heads per token (0: ngroups) with
    ``norm_eps``.
    """
    Bt, L, H, P, N, G = _check_scan_inputs(x, dt, A, B, C, D)
    dev = x.device
    if init_state is not None:
        _need(init_state, "init_state", (Bt, H, P, N), torch.float32, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", (Bt, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, x.dtype, dev)
    desc = _scan_desc(x, B, chunk)
    n = ctypes.c_size_t(0)
    _check("ssd_scan_workspace_size", lib().ssd_scan_workspace_size(ctypes.byref(desc),
                                                                    ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < n.value or workspace.device != dev:
        raise ValueError(f"workspace needs {n.value} bytes on {dev}")
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    st = lib().ssd_scan_fwd_ex(ctypes.byref(desc), _eref(e), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    _check("ssd_scan_fwd_ex", st)
    return y, final_state


def scan_bwd(x, dt, A, B, C, dy, D=None, init_state=None, dfinal=None, chunk: int = 256,
             workspace=None, dt_bias=None, dt_softplus: bool = False, dt_limit=None,
             z=None, norm_weight=None, norm_eps: float = 1e-5, norm_groups: int = 0) -> dict:
    """Gradient of :func:`scan_fwd`: derivatives of sum(dy * y) + sum(dfinal *
    final_state) with respect to x, dt, A, B, C, D and init_state.  Returns a
    dict: dx (x's dtype), ddt, dA, dB, dC (fp32), dD (None without D) and
    dinit (None without init_state and dfinal).

    With the fused edges of :func:`scan_fwd` (``dt_bias``, ``dt_softplus``,
    ``dt_limit``, gate ``z``, gated RMSNorm ``norm_weight``), dt is the raw
    step size and ddt its gradient; the dict also holds ``dz`` (with z),
    ``ddt_bias`` (with dt_bias) and ``dnorm_weight`` (with norm_weight)."""
    Bt, L, H, P, N, G = _check_scan_inputs(x, dt, A, B, C, D)
    dev = x.device
    _need(dy, "dy", x.shape, x.dtype, dev)
    if init_state is not None:
        _need(init_state, "init_state", (Bt, H, P, N), torch.float32, dev)
    if dfinal is not None:
        _need(dfinal, "dfinal", (Bt, H, P, N), torch.float32, dev)
    desc = _scan_desc(x, B, chunk)
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    n = ctypes.c_size_t(0)
    _check("ssd_scan_bwd_ex_workspace_size",
           lib().ssd_scan_bwd_ex_workspace_size(ctypes.byref(desc), _eref(e), ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < n.value or workspace.device != dev:
        raise ValueError(f"workspace needs {n.value} bytes on {dev}")
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty((Bt, L, H), **f32),
           "dA": torch.empty(H, **f32), "dB": torch.empty((Bt, L, G, N), **f32),
           "dC": torch.empty((Bt, L, G, N), **f32),
           "dD": torch.empty(H, **f32) if D is not None else None,
           "dinit": (torch.empty((Bt, H, P, N), **f32)
                     if init_state is not None or dfinal is not None else None)}
    if z is not None:
        out["dz"] = torch.empty_like(x)
    if dt_bias is not None:
        out["ddt_bias"] = torch.empty(H, **f32)
    if norm_weight is not None:
        out["dnorm_weight"] = torch.empty(H * P, **f32)
    st = lib().ssd_scan_bwd_ex(ctypes.byref(desc), _eref(e), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(init_state), _ptr(dy), _ptr(dfinal),
                               _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
                               _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                               _ptr(out["dinit"]), _ptr(out.get("dz")),
                               _ptr(out.get("ddt_bias")), _ptr(out.get("dnorm_weight")),
                               _ptr(workspace), workspace.numel(),
                               _stream(dev))
    _check("ssd_scan_bwd_ex", st)
    return out


def scan_bwd_varlen(x, dt, A, B, C, cu_seqlens, dy, D=None, chunk: int = 256,
                    init_states=None, dfinal_states=None, workspace=None, dt_bias=None,
                    dt_softplus: bool = False, dt_limit=None, z=None, norm_weight=None,
                    norm_eps: float = 1e-5, norm_groups: int = 0) -> dict:
    """Gradient of :func:`scan_fwd_varlen` (edges as for :func:`scan_bwd`):
    every sequence's own gradient.  Returns a dict like scan_bwd's, with dinit
    per sequence [nseq, nheads, headdim, dstate]."""
    if x.dim() != 3 or B.dim() != 3 or dt.dim() != 2:
        raise ValueError("x [total,h,p], dt [total,h], B/C [total,g,n] expected")
    total, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    ns = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (ns + 1,), torch.int32, dev)
    _need(dy, "dy", x.shape, x.dtype, dev)
    if init_states is not None:
        _need(init_states, "init_states", (ns, H, P, N), torch.float32, dev)
    if dfinal_states is not None:
        _need(dfinal_states, "dfinal_states", (ns, H, P, N), torch.float32, dev)
    desc = VarlenDesc(ns, total, H, P, N, G, chunk, _io_dtype(x), 0)
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    n = ctypes.c_size_t(0)
    _check("ssd_scan_bwd_varlen_workspace_size",
           lib().ssd_scan_bwd_varlen_workspace_size(ctypes.byref(desc), _eref(e),
                                                    ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < n.value or workspace.device != dev:
        raise ValueError(f"workspace needs {n.value} bytes on {dev}")
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty((total, H), **f32),
           "dA": torch.empty(H, **f32), "dB": torch.empty((total, G, N), **f32),
           "dC": torch.empty((total, G, N), **f32),
           "dD": torch.empty(H, **f32) if D is not None else None,
           "dinit": (torch.empty((ns, H, P, N), **f32)
                     if init_states is not None or dfinal_states is not None else None)}
    if z is not None:
        out["dz"] = torch.empty_like(x)
    if dt_bias is not None:
        out["ddt_bias"] = torch.empty(H, **f32)
    if norm_weight is not None:
        out["dnorm_weight"] = torch.empty(H * P, **f32)
    st = lib().ssd_scan_bwd_varlen(
        ctypes.byref(desc), _eref(e), _ptr(cu_seqlens), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
        _ptr(C), _ptr(D), _ptr(init_states), _ptr(dy), _ptr(dfinal_states), _ptr(out["dx"]),
        _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
        _ptr(out["dinit"]), _ptr(out.get("dz")), _ptr(out.get("ddt_bias")),
        _ptr(out.get("dnorm_weight")), _ptr(workspace), workspace.numel(), _stream(dev))
    _check("ssd_scan_bwd_varlen", st)
    return out


def varlen_workspace_size(nseq, total, nheads, headdim, dstate, ngroups, chunk, dtype) -> int:
    d = VarlenDesc(nseq, total, nheads, headdim, dstate, ngroups, chunk,
                   SSD_BF16 if dtype == torch.bfloat16 else SSD_F32, 0)
    n = ctypes.c_size_t(0)
    _check("ssd_varlen_workspace_size",
           lib().ssd_varlen_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def scan_fwd_varlen(x, dt, A, B, C, cu_seqlens, D=None, chunk: int = 256, init_states=None,
                    return_final_states: bool = True, final_states=None, workspace=None,
                    y=None, dt_bias=None, dt_softplus: bool = False, dt_limit=None, z=None,
                    norm_weight=None, norm_eps: float = 1e-5, norm_groups: int = 0):
    """Ragged batch: sequence s is tokens [cu_seqlens[s], cu_seqlens[s+1]) of
    the packed x [total, nheads, headdim], dt [total, nheads], B/C [total,
    ngroups, dstate]; cu_seqlens is an int32 device tensor [nseq + 1].
    Returns (y, final_states [nseq, nheads, headdim, dstate] or None)."""
    if x.dim() != 3 or B.dim() != 3 or dt.dim() != 2:
        raise ValueError("x [total,h,p], dt [total,h], B/C [total,g,n] expected")
    total, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev, io = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be device tensors")
    if cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor [nseq + 1]")
    nseq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int32, dev)
    _need(dt, "dt", (total, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (total, G, N), io, dev)
    _need(C, "C", (total, G, N), io, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (nseq, H, P, N), torch.float32, dev)
    if final_states is None and return_final_states:
        final_states = torch.empty((nseq, H, P, N), dtype=torch.float32, device=dev)
    elif final_states is not None:
        _need(final_states, "final_states", (nseq, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, io, dev)
    desc = VarlenDesc(nseq, total, H, P, N, G, chunk, _io_dtype(x), 0)
    n = ctypes.c_size_t(0)
    _check("ssd_varlen_workspace_size",
           lib().ssd_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < n.value or workspace.device != dev:
        raise ValueError(f"workspace needs {n.value} bytes on {dev}")
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    st = lib().ssd_scan_fwd_varlen(ctypes.byref(desc), _eref(e), _ptr(cu_seqlens), _ptr(x),
                                   _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(init_states), _ptr(y), _ptr(final_states),
                                   _ptr(workspace), workspace.numel(), _stream(dev))
    _check("ssd_scan_fwd_varlen", st)
    return y, final_states


def step(state, x, dt, A, B, C, D=None, y=None, dt_bias=None, dt_softplus: bool = False,
         dt_limit=None, z=None, norm_weight=None, norm_eps: float = 1e-5, norm_groups: int = 0):
    """One decode token; ``state`` [batch, nheads, headdim, dstate] fp32 is updated in place.
    Fused edges as for :func:`scan_fwd` (``z`` has x's shape)."""
    if state.dim() != 4 or x.dim() != 3 or B.dim() != 3:
        raise ValueError("state [b,h,p,n], x [b,h,p], B/C [b,g,n] expected")
    Bt, H, P, N = state.shape
    G = B.shape[1]
    dev, io = state.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be device tensors")
    _need(state, "state", (Bt, H, P, N), torch.float32, dev)
    _need(x, "x", (Bt, H, P), io, dev)
    _need(dt, "dt", (Bt, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (Bt, G, N), io, dev)
    _need(C, "C", (Bt, G, N), io, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, io, dev)
    desc = StepDesc(Bt, H, P, N, G, _io_dtype(x), 0)
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    st = lib().ssd_step_ex(ctypes.byref(desc), _eref(e), _ptr(state), _ptr(x), _ptr(dt), _ptr(A),
                           _ptr(B), _ptr(C), _ptr(D), _ptr(y), _stream(dev))
    _check("ssd_step_ex", st)
    return y


def step_multi(state, x, dt, A, B, C, D=None, y=None, dt_bias=None, dt_softplus: bool = False,
               dt_limit=None, z=None, norm_weight=None, norm_eps: float = 1e-5,
               norm_groups: int = 0):
    """nsteps decode tokens in one launch (inputs in the prefill layout: x
    [batch, nsteps, nheads, headdim], dt [batch, nsteps, nheads], B/C
    [batch, nsteps, ngroups, dstate]); ``state`` is updated in place.  Equal to
    nsteps calls of :func:`step` (fused edges likewise)."""
    if state.dim() != 4 or x.dim() != 4 or B.dim() != 4:
        raise ValueError("state [b,h,p,n], x [b,t,h,p], B/C [b,t,g,n] expected")
    Bt, H, P, N = state.shape
    T, G = x.shape[1], B.shape[2]
    dev, io = state.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be device tensors")
    _need(state, "state", (Bt, H, P, N), torch.float32, dev)
    _need(x, "x", (Bt, T, H, P), io, dev)
    _need(dt, "dt", (Bt, T, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (Bt, T, G, N), io, dev)
    _need(C, "C", (Bt, T, G, N), io, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, io, dev)
    desc = StepDesc(Bt, H, P, N, G, _io_dtype(x), 0)
    e = _edges(x, H, P, dt_bias, dt_softplus, dt_limit, z, norm_weight, norm_eps, norm_groups)
    st = lib().ssd_step_multi_ex(ctypes.byref(desc), _eref(e), T, _ptr(state), _ptr(x), _ptr(dt),
                                 _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y), _stream(dev))
    _check("ssd_step_multi_ex", st)
    return y


def chunk_cumsum(dt, A, chunk: int, x_like):
    """Stage 1: Acs [batch, nheads, seqlen] fp32.  ``x_like`` gives the shape/dtype desc."""
    x, B = x_like
    desc = _scan_desc(x, B, chunk)
    Bt, L, H = dt.shape
    _need(dt, "dt", (Bt, L, H), torch.float32, x.device)
    _need(A, "A", (H,), torch.float32, x.device)
    Acs = torch.empty((Bt, H, L), dtype=torch.float32, device=x.device)
    _check("ssd_chunk_cumsum", lib().ssd_chunk_cumsum(ctypes.byref(desc), _ptr(dt), _ptr(A),
                                                      _ptr(Acs), _stream(x.device)))
    return Acs


def chunk_state(x, B, dt, Acs, chunk: int):
    """Stage 2: states [batch, T, nheads, headdim, dstate] fp32 (each chunk alone)."""
    Bt, L, H, P, N, G = _check_scan_inputs(x, dt, torch.empty(x.shape[2], device=x.device),
                                           B, None, None)
    _need(Acs, "Acs", (Bt, H, L), torch.float32, x.device)
    T = -(-L // chunk)
    states = torch.empty((Bt, T, H, P, N), dtype=torch.float32, device=x.device)
    desc = _scan_desc(x, B, chunk)
    _check("ssd_chunk_state", lib().ssd_chunk_state(ctypes.byref(desc), _ptr(x), _ptr(B),
                                                    _ptr(dt), _ptr(Acs), _ptr(states),
                                                    _stream(x.device)))
    return states


def state_passing(states, Acs, chunk: int, x_like, init_state=None, final_state=None):
    """Stage 3, in place: states[c] becomes the state entering chunk c.  Returns final_state."""
    x, B = x_like
    Bt, L, H, P = x.shape
    N = B.shape[3]
    T = -(-L // chunk)
    dev = x.device
    _need(states, "states", (Bt, T, H, P, N), torch.float32, dev)
    _need(Acs, "Acs", (Bt, H, L), torch.float32, dev)
    if init_state is not None:
        _need(init_state, "init_state", (Bt, H, P, N), torch.float32, dev)
    if final_state is None:
        final_state = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
    desc = _scan_desc(x, B, chunk)
    _check("ssd_state_passing", lib().ssd_state_passing(ctypes.byref(desc), _ptr(states),
                                                        _ptr(Acs), _ptr(init_state),
                                                        _ptr(final_state), _stream(dev)))
    return final_state


def chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                              dtype) -> int:
    d = ScanDesc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                 SSD_BF16 if dtype == torch.bfloat16 else SSD_F32, 0)
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_scan_workspace_size",
           lib().ssd_chunk_scan_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def chunk_cb(x, B, C, chunk: int, workspace=None):
    """Stage: the within-chunk C.B products of every (batch, chunk, group)
    into a uint8 device workspace (returned; None when the shape needs none).
    ``x`` only supplies the shape and dtype of the call."""
    Bt, L, H, P, N, G = _check_scan_inputs(x, torch.empty(x.shape[:3], device=x.device),
                                           torch.empty(x.shape[2], device=x.device), B, C, None)
    desc = _scan_desc(x, B, chunk)
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_scan_workspace_size",
           lib().ssd_chunk_scan_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    if n.value == 0:
        return None
    if workspace is None:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("ssd_chunk_cb", lib().ssd_chunk_cb(ctypes.byref(desc), _ptr(B), _ptr(C),
                                              _ptr(workspace), ws_bytes, _stream(x.device)))
    return workspace


def chunk_scan(x, dt, B, C, D, Acs, states, chunk: int, workspace=None):
    """Stage: y from the chunk-entry states.  ``workspace`` is what
    :func:`chunk_cb` returned for the same B and C; when omitted it is formed
    here first."""
    Bt, L, H, P, N, G = _check_scan_inputs(x, dt, torch.empty(x.shape[2], device=x.device),
                                           B, C, D)
    T = -(-L // chunk)
    _need(Acs, "Acs", (Bt, H, L), torch.float32, x.device)
    _need(states, "states", (Bt, T, H, P, N), torch.float32, x.device)
    if workspace is None:
        workspace = chunk_cb(x, B, C, chunk)
    y = torch.empty_like(x)
    desc = _scan_desc(x, B, chunk)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ssd_chunk_scan", lib().ssd_chunk_scan(ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(B),
                                                  _ptr(C), _ptr(D), _ptr(Acs), _ptr(states),
                                                  _ptr(y), _ptr(workspace), ws_bytes,
                                                  _stream(x.device)))
    return y
