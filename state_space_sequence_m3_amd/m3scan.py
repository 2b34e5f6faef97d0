"""ctypes binding of libm3scan with the same entry-point names as the C ABI (include/m3scan.h).

This module only marshals arguments: it checks tensor placement, dtype, shape and contiguity,
allocates outputs and workspaces with torch when the caller does not pass them, passes raw
device pointers and the current HIP stream, and turns a non-OK status into an exception.  Every
step of the computation runs in the library's HIP kernels.  There is no fallback: if
``libm3scan.so`` is not built, or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm3scan.so")

M3_OK, M3_E_NULL, M3_E_DIMS, M3_E_ALIGN, M3_E_DTYPE = 0, 1, 2, 3, 4
M3_E_UNSUPPORTED, M3_E_NODEVICE, M3_E_LAUNCH, M3_E_WORKSPACE, M3_E_ALIAS = 5, 6, 7, 8, 9
STATUS_NAMES = {0: "M3_OK", 1: "M3_E_NULL", 2: "M3_E_DIMS", 3: "M3_E_ALIGN", 4: "M3_E_DTYPE",
                5: "M3_E_UNSUPPORTED", 6: "M3_E_NODEVICE", 7: "M3_E_LAUNCH", 8: "M3_E_WORKSPACE",
                9: "M3_E_ALIAS"}
M3_F32, M3_BF16 = 0, 1
M3_BCNORM = 1

EXPORTED = ["m3_bcnorm_rope", "m3_bcnorm_rope_workspace_bytes", "m3_prefill",
            "m3_prefill_workspace_bytes", "m3_layer_prefill", "m3_layer_prefill_workspace_bytes",
            "m3_layer_prefill_varlen",
            "m3_decode_step",
            "m3_layer_decode_step", "m3_layer_backward_chunk", "m3_layer_chunk_states",
            "m3_layer_backward_workspace_bytes", "m3_layer_backward", "m3_last_error", "m3_version",
            "m3_layer_prefill_noalloc"]
NOALLOC_SCRATCH_BYTES = 32 << 20   # M3_NOALLOC_SCRATCH_BYTES


class M3Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("eps", ctypes.c_float), ("ngroups", ctypes.c_int64)]


class M3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_DIMS = ctypes.POINTER(M3Dims)


def load(path: str = LIB_PATH):
    """Load libm3scan.so (once) and declare the C signatures.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("libm3scan.so is not built (%s); run "
                                   "`python -m state_space_sequence_m3_amd.build`" % path)
            lib = ctypes.CDLL(path)
            lib.m3_bcnorm_rope.restype = ctypes.c_int
            lib.m3_bcnorm_rope.argtypes = [_DIMS] + [_P] * 13 + [ctypes.c_size_t, _P]
            lib.m3_bcnorm_rope_workspace_bytes.restype = ctypes.c_size_t
            lib.m3_bcnorm_rope_workspace_bytes.argtypes = [_DIMS]
            lib.m3_prefill.restype = ctypes.c_int
            lib.m3_prefill.argtypes = [_DIMS] + [_P] * 15 + [ctypes.c_size_t, _P]
            lib.m3_prefill_workspace_bytes.restype = ctypes.c_size_t
            lib.m3_prefill_workspace_bytes.argtypes = [_DIMS]
            lib.m3_layer_prefill_workspace_bytes.restype = ctypes.c_size_t
            lib.m3_layer_prefill_workspace_bytes.argtypes = [_DIMS]
            lib.m3_layer_prefill.restype = ctypes.c_int
            lib.m3_layer_prefill.argtypes = [_DIMS] + [_P] * 22 + [ctypes.c_size_t, _P]
            lib.m3_layer_prefill_noalloc.restype = ctypes.c_int
            lib.m3_layer_prefill_noalloc.argtypes = [_DIMS] + [_P] * 21 + [_P]
            lib.m3_layer_prefill_varlen.restype = ctypes.c_int
            lib.m3_layer_prefill_varlen.argtypes = [_DIMS] + [_P] * 22 + [_P]
            lib.m3_layer_decode_step.restype = ctypes.c_int
            lib.m3_layer_decode_step.argtypes = [_DIMS] + [_P] * 18 + [_P]
            lib.m3_decode_step.restype = ctypes.c_int
            lib.m3_decode_step.argtypes = [_DIMS] + [_P] * 11 + [_P]
            lib.m3_layer_backward_chunk.restype = ctypes.c_int64
            lib.m3_layer_backward_chunk.argtypes = [_DIMS]
            lib.m3_layer_chunk_states.restype = ctypes.c_int
            lib.m3_layer_chunk_states.argtypes = [_DIMS] + [_P] * 14 + [_P]
            lib.m3_layer_backward_workspace_bytes.restype = ctypes.c_size_t
            lib.m3_layer_backward_workspace_bytes.argtypes = [_DIMS]
            lib.m3_layer_backward.restype = ctypes.c_int
            lib.m3_layer_backward.argtypes = [_DIMS] + [_P] * 36 + [ctypes.c_size_t, _P]
            lib.m3_last_error.restype = ctypes.c_char_p
            lib.m3_last_error.argtypes = []
            lib.m3_version.restype = ctypes.c_char_p
            lib.m3_version.argtypes = []
            _lib = lib
    return _lib


def version() -> str:
    return load().m3_version().decode()


def last_error() -> str:
    return load().m3_last_error().decode()


def _check(status: int):
    if status != M3_OK:
        raise M3Error(status, last_error())


def _io_code(dtype) -> int:
    if dtype == torch.float32:
        return M3_F32
    if dtype == torch.bfloat16:
        return M3_BF16
    raise ValueError("io tensors must be float32 or bfloat16, got %s" % dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _tensor(t, name, shape, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def make_dims(batch, seqlen, nheads, headdim, dstate, rank, chunk=0, io=M3_BF16, bcnorm=True,
              eps=1e-5, groups=0) -> M3Dims:
    """``groups`` = G head slots of raw B and C (heads share them in groups of H / G); 0 = one
    per head."""
    return M3Dims(batch, seqlen, nheads, headdim, dstate, rank, chunk, io,
                  M3_BCNORM if bcnorm else 0, eps, groups)


def _groups(H, G):
    """The dims field for raw B and C with G head slots and H heads (0 when G == H)."""
    if G < 1 or H % G != 0:
        raise ValueError("B and C have %d head slots, which must divide the %d heads" % (G, H))
    return 0 if G == H else G


def bcnorm_rope_workspace_bytes(dims: M3Dims) -> int:
    return int(load().m3_bcnorm_rope_workspace_bytes(ctypes.byref(dims)))


def prefill_workspace_bytes(dims: M3Dims) -> int:
    return int(load().m3_prefill_workspace_bytes(ctypes.byref(dims)))


def layer_prefill_workspace_bytes(dims: M3Dims) -> int:
    return load().m3_layer_prefill_workspace_bytes(ctypes.byref(dims))


def m3_bcnorm_rope(B, C, dt, theta, normw_B=None, normw_C=None, bias_B=None, bias_C=None,
                   phi_in=None, Bbar=None, Cbar=None, phi_out=None, bcnorm=True, eps=1e-5,
                   workspace=None, stream=None):
    """BCNorm + bias + cumulative rotation.  B, C: [b, L, G, R, N] raw (G = H, or head slots
    shared by groups of H / G heads; H is taken from dt); returns (Bbar, Cbar, phi_out) with
    Bbar, Cbar [b, L, H, R, N]."""
    lib = load()
    b, L, G, R, N = B.shape
    H = dt.shape[2]
    dev, io = B.device, B.dtype
    f32 = torch.float32
    _tensor(B, "B", (b, L, G, R, N), io, dev)
    _tensor(C, "C", (b, L, G, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(theta, "theta", (b, L, H, N // 2), io, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    oshape = (b, L, H, R, N)
    Bbar = torch.empty(oshape, dtype=io, device=dev) if Bbar is None else _tensor(Bbar, "Bbar", oshape, io, dev)
    Cbar = torch.empty(oshape, dtype=io, device=dev) if Cbar is None else _tensor(Cbar, "Cbar", oshape, io, dev)
    if phi_out is None:
        phi_out = torch.empty((b, H, N // 2), dtype=f32, device=dev)
    _tensor(phi_out, "phi_out", (b, H, N // 2), f32, dev)
    dims = make_dims(b, L, H, 0, N, R, 0, _io_code(io), bcnorm, eps, _groups(H, G))
    need = bcnorm_rope_workspace_bytes(dims)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m3_bcnorm_rope(ctypes.byref(dims), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                              _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C),
                              _ptr(phi_in), _ptr(Bbar), _ptr(Cbar), _ptr(phi_out),
                              _ptr(workspace), ws_bytes, _stream(stream)))
    return Bbar, Cbar, phi_out


def _workspace(workspace, need, dev):
    """A prefill call's workspace: None allocates the bytes the library asks for (it then splits
    few long sequences into segments), False passes none (one pass per sequence), a tensor is
    used as given.  Returns (tensor or None, bytes)."""
    if workspace is False:
        return None, 0
    if workspace is None:
        if not need:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def m3_prefill(x, Bbar, Cbar, dt, A, lam, w_out=None, h_in=None, Bbar_prev=None, x_prev=None,
               y=None, h_out=None, Bbar_last=None, x_last=None, chunk=0, workspace=None,
               stream=None):
    """Chunked scan.  x: [b, L, H, R, P]; Bbar, Cbar: [b, L, H, R, N].  Returns (y, h_out)."""
    lib = load()
    b, L, H, R, P = x.shape
    N = Bbar.shape[-1]
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(Bbar, "Bbar", (b, L, H, R, N), io, dev)
    _tensor(Cbar, "Cbar", (b, L, H, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(lam, "lam", (b, L, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    yshape = (b, L, H, P) if w_out is not None else (b, L, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    if h_out is None:
        h_out = torch.empty((b, H, N, P), dtype=f32, device=dev)
    _tensor(h_out, "h_out", (b, H, N, P), f32, dev)
    _tensor(Bbar_last, "Bbar_last", (b, H, R, N), io, dev)
    _tensor(x_last, "x_last", (b, H, R, P), io, dev)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(io))
    workspace, ws_bytes = _workspace(workspace, prefill_workspace_bytes(dims), dev)
    _check(lib.m3_prefill(ctypes.byref(dims), _ptr(x), _ptr(Bbar), _ptr(Cbar), _ptr(dt), _ptr(A),
                          _ptr(lam), _ptr(w_out), _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev),
                          _ptr(y), _ptr(h_out), _ptr(Bbar_last), _ptr(x_last), _ptr(workspace),
                          ws_bytes, _stream(stream)))
    return y, h_out


def m3_layer_prefill(x, B, C, dt, theta, A, lam, normw_B=None, normw_C=None, bias_B=None,
                     bias_C=None, w_out=None, phi_in=None, h_in=None, Bbar_prev=None, x_prev=None,
                     y=None, h_out=None, phi_out=None, Bbar_last=None, x_last=None, chunk=0,
                     bcnorm=True, eps=1e-5, workspace=None, stream=None):
    """m3_bcnorm_rope + m3_prefill in one pass.  x: [b, L, H, R, P]; raw B, C: [b, L, G, R, N]
    (G = H, or head slots shared by groups of H / G heads).  A workspace of
    layer_prefill_workspace_bytes is allocated when none is given (it lets few long sequences
    run split into segments).  Returns (y, h_out, phi_out)."""
    lib = load()
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[-1]
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(B, "B", (b, L, G, R, N), io, dev)
    _tensor(C, "C", (b, L, G, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(theta, "theta", (b, L, H, N // 2), io, dev)
    _tensor(lam, "lam", (b, L, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    yshape = (b, L, H, P) if w_out is not None else (b, L, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    if h_out is None:
        h_out = torch.empty((b, H, N, P), dtype=f32, device=dev)
    _tensor(h_out, "h_out", (b, H, N, P), f32, dev)
    if phi_out is None:
        phi_out = torch.empty((b, H, N // 2), dtype=f32, device=dev)
    _tensor(phi_out, "phi_out", (b, H, N // 2), f32, dev)
    _tensor(Bbar_last, "Bbar_last", (b, H, R, N), io, dev)
    _tensor(x_last, "x_last", (b, H, R, P), io, dev)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(io), bcnorm, eps, _groups(H, G))
    workspace, ws_bytes = _workspace(workspace, layer_prefill_workspace_bytes(dims), dev)
    _check(lib.m3_layer_prefill(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                                _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C), _ptr(A),
                                _ptr(lam), _ptr(w_out), _ptr(phi_in), _ptr(h_in), _ptr(Bbar_prev),
                                _ptr(x_prev), _ptr(y), _ptr(h_out), _ptr(phi_out), _ptr(Bbar_last),
                                _ptr(x_last), _ptr(workspace), ws_bytes, _stream(stream)))
    return y, h_out, phi_out


def m3_layer_prefill_noalloc(x, B, C, dt, theta, A, lam, normw_B=None, normw_C=None, bias_B=None,
                             bias_C=None, w_out=None, phi_in=None, h_in=None, Bbar_prev=None,
                             x_prev=None, y=None, h_out=None, phi_out=None, Bbar_last=None,
                             x_last=None, chunk=0, bcnorm=True, eps=1e-5, stream=None):
    """m3_layer_prefill without a workspace argument: a split of few long sequences uses the
    library's own device scratch array (M3_NOALLOC_SCRATCH_BYTES per GPU).  The library itself
    allocates nothing; outputs not passed are allocated here (pass them all for an allocation-free
    call).  Returns (y, h_out, phi_out)."""
    lib = load()
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[-1]
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(B, "B", (b, L, G, R, N), io, dev)
    _tensor(C, "C", (b, L, G, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(theta, "theta", (b, L, H, N // 2), io, dev)
    _tensor(lam, "lam", (b, L, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    yshape = (b, L, H, P) if w_out is not None else (b, L, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    if h_out is None:
        h_out = torch.empty((b, H, N, P), dtype=f32, device=dev)
    _tensor(h_out, "h_out", (b, H, N, P), f32, dev)
    if phi_out is None:
        phi_out = torch.empty((b, H, N // 2), dtype=f32, device=dev)
    _tensor(phi_out, "phi_out", (b, H, N // 2), f32, dev)
    _tensor(Bbar_last, "Bbar_last", (b, H, R, N), io, dev)
    _tensor(x_last, "x_last", (b, H, R, P), io, dev)
    dims = make_dims(b, L, H, P, N, R, chunk, _io_code(io), bcnorm, eps, _groups(H, G))
    _check(lib.m3_layer_prefill_noalloc(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                                        _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C), _ptr(A),
                                        _ptr(lam), _ptr(w_out), _ptr(phi_in), _ptr(h_in), _ptr(Bbar_prev),
                                        _ptr(x_prev), _ptr(y), _ptr(h_out), _ptr(phi_out), _ptr(Bbar_last),
                                        _ptr(x_last), _stream(stream)))
    return y, h_out, phi_out


def m3_decode_step(h, Bbar_prev, x_prev, x, Bbar, Cbar, dt, A, lam, w_out=None, y=None,
                   stream=None):
    """One decode token, state h [b, H, N, P] updated in place.  Returns y."""
    lib = load()
    b, H, N, P = h.shape
    R = x.shape[2]
    dev, io = h.device, x.dtype
    f32 = torch.float32
    _tensor(h, "h", (b, H, N, P), f32, dev)
    for name, t, shp in (("Bbar_prev", Bbar_prev, (b, H, R, N)), ("x_prev", x_prev, (b, H, R, P)),
                         ("x", x, (b, H, R, P)), ("Bbar", Bbar, (b, H, R, N)),
                         ("Cbar", Cbar, (b, H, R, N)), ("dt", dt, (b, H)), ("lam", lam, (b, H))):
        _tensor(t, name, shp, io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    yshape = (b, H, P) if w_out is not None else (b, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    dims = make_dims(b, 1, H, P, N, R, 0, _io_code(io))
    _check(lib.m3_decode_step(ctypes.byref(dims), _ptr(h), _ptr(Bbar_prev), _ptr(x_prev), _ptr(x),
                              _ptr(Bbar), _ptr(Cbar), _ptr(dt), _ptr(A), _ptr(lam), _ptr(w_out),
                              _ptr(y), _stream(stream)))
    return y


def m3_layer_decode_step(h, phi, Bbar_prev, x_prev, x, B, C, dt, theta, A, lam, normw_B=None,
                         normw_C=None, bias_B=None, bias_C=None, w_out=None, y=None, Bbar_out=None,
                         bcnorm=True, eps=1e-5, stream=None):
    """Rotation + one decode token: h [b, H, N, P] and phi [b, H, N/2] updated in place; raw B,
    C [b, G, R, N] (G = H, or head slots shared by groups of H / G heads).
    Returns (y, Bbar_out); Bbar_out [b, H, R, N] is the next step's Bbar_prev."""
    lib = load()
    b, H, N, P = h.shape
    R = x.shape[2]
    G = B.shape[1]
    dev, io = h.device, x.dtype
    f32 = torch.float32
    _tensor(h, "h", (b, H, N, P), f32, dev)
    _tensor(phi, "phi", (b, H, N // 2), f32, dev)
    for name, t, shp in (("Bbar_prev", Bbar_prev, (b, H, R, N)), ("x_prev", x_prev, (b, H, R, P)),
                         ("x", x, (b, H, R, P)), ("B", B, (b, G, R, N)), ("C", C, (b, G, R, N)),
                         ("dt", dt, (b, H)), ("theta", theta, (b, H, N // 2)), ("lam", lam, (b, H))):
        _tensor(t, name, shp, io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    yshape = (b, H, P) if w_out is not None else (b, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    if Bbar_out is None:
        Bbar_out = torch.empty((b, H, R, N), dtype=io, device=dev)
    _tensor(Bbar_out, "Bbar_out", (b, H, R, N), io, dev)
    dims = make_dims(b, 1, H, P, N, R, 0, _io_code(io), bcnorm, eps, _groups(H, G))
    _check(lib.m3_layer_decode_step(ctypes.byref(dims), _ptr(h), _ptr(phi), _ptr(Bbar_prev),
                                    _ptr(x_prev), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta),
                                    _ptr(normw_B), _ptr(normw_C), _ptr(bias_B), _ptr(bias_C),
                                    _ptr(A), _ptr(lam), _ptr(w_out), _ptr(y), _ptr(Bbar_out),
                                    _stream(stream)))
    return y, Bbar_out


def m3_layer_prefill_varlen(cu_seqlens, x, B, C, dt, theta, A, lam, normw_B=None, normw_C=None,
                            bias_B=None, bias_C=None, w_out=None, phi_in=None, h_in=None,
                            Bbar_prev=None, x_prev=None, y=None, h_out=None, phi_out=None,
                            Bbar_last=None, x_last=None, chunk=0, bcnorm=True, eps=1e-5, stream=None):
    """m3_layer_prefill over a packed batch: x [T, H, R, P], B, C [T, G, R, N], ...; sequence s is
    tokens cu_seqlens[s]:cu_seqlens[s+1] (int32 device tensor of b + 1 offsets).
    Returns (y, h_out, phi_out)."""
    lib = load()
    T, H, R, P = x.shape
    G, N = B.shape[1], B.shape[-1]
    b = cu_seqlens.numel() - 1
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(cu_seqlens, "cu_seqlens", (b + 1,), torch.int32, dev)
    _tensor(B, "B", (T, G, R, N), io, dev)
    _tensor(C, "C", (T, G, R, N), io, dev)
    _tensor(dt, "dt", (T, H), io, dev)
    _tensor(theta, "theta", (T, H, N // 2), io, dev)
    _tensor(lam, "lam", (T, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    yshape = (T, H, P) if w_out is not None else (T, H, R, P)
    y = torch.empty(yshape, dtype=io, device=dev) if y is None else _tensor(y, "y", yshape, io, dev)
    if h_out is None:
        h_out = torch.empty((b, H, N, P), dtype=f32, device=dev)
    _tensor(h_out, "h_out", (b, H, N, P), f32, dev)
    if phi_out is None:
        phi_out = torch.empty((b, H, N // 2), dtype=f32, device=dev)
    _tensor(phi_out, "phi_out", (b, H, N // 2), f32, dev)
    _tensor(Bbar_last, "Bbar_last", (b, H, R, N), io, dev)
    _tensor(x_last, "x_last", (b, H, R, P), io, dev)
    dims = make_dims(b, T, H, P, N, R, chunk, _io_code(io), bcnorm, eps, _groups(H, G))
    _check(lib.m3_layer_prefill_varlen(ctypes.byref(dims), _ptr(cu_seqlens), _ptr(x), _ptr(B), _ptr(C),
                                       _ptr(dt), _ptr(theta), _ptr(normw_B), _ptr(normw_C), _ptr(bias_B),
                                       _ptr(bias_C), _ptr(A), _ptr(lam), _ptr(w_out), _ptr(phi_in),
                                       _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev), _ptr(y), _ptr(h_out),
                                       _ptr(phi_out), _ptr(Bbar_last), _ptr(x_last), _stream(stream)))
    return y, h_out, phi_out


def layer_backward_chunk(dims: M3Dims) -> int:
    """Time steps per chunk of the backward pass (0 when unsupported)."""
    return int(load().m3_layer_backward_chunk(ctypes.byref(dims)))


def layer_backward_workspace_bytes(dims: M3Dims) -> int:
    return int(load().m3_layer_backward_workspace_bytes(ctypes.byref(dims)))


def m3_layer_chunk_states(x, B, dt, theta, A, lam, normw_B=None, bias_B=None, phi_in=None, h_in=None,
                          Bbar_prev=None, x_prev=None, states=None, phis=None, bcnorm=True, eps=1e-5,
                          stream=None):
    """Entry state and angle of every backward chunk (raw B: [b, L, G, R, N]).  Returns (states
    [b, H, nchunk, P, N] io, phis [b, H, nchunk, N/2] f32) and the chunk length in steps."""
    lib = load()
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[-1]
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(B, "B", (b, L, G, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(theta, "theta", (b, L, H, N // 2), io, dev)
    _tensor(lam, "lam", (b, L, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    dims = make_dims(b, L, H, P, N, R, 0, _io_code(io), bcnorm, eps, _groups(H, G))
    Q = layer_backward_chunk(dims)
    if Q == 0:
        raise M3Error(M3_E_UNSUPPORTED, "no backward kernel for N=%d P=%d R=%d" % (N, P, R))
    nc = (L + Q - 1) // Q
    if states is None:
        states = torch.empty((b, H, nc, P, N), dtype=io, device=dev)
    _tensor(states, "states", (b, H, nc, P, N), io, dev)
    if phis is None:
        phis = torch.empty((b, H, nc, N // 2), dtype=f32, device=dev)
    _tensor(phis, "phis", (b, H, nc, N // 2), f32, dev)
    _check(lib.m3_layer_chunk_states(ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(dt), _ptr(theta),
                                     _ptr(normw_B), _ptr(bias_B), _ptr(A), _ptr(lam), _ptr(phi_in),
                                     _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev), _ptr(states),
                                     _ptr(phis), _stream(stream)))
    return states, phis, Q


def m3_layer_backward(x, B, C, dt, theta, A, lam, dy, normw_B=None, normw_C=None, bias_B=None,
                      bias_C=None, w_out=None, phi_in=None, h_in=None, Bbar_prev=None, x_prev=None,
                      dh_out=None, dphi_out=None, grads=None, bcnorm=True, eps=1e-5, workspace=None,
                      stream=None):
    """Gradients of m3_layer_prefill.  ``dy`` has y's shape; dh_out [b, H, N, P] and dphi_out
    [b, H, N/2] are optional (zero).  Returns a dict keyed by input name (x, B, C, dt, theta, A,
    lam, normw_B, normw_C, bias_B, bias_C, w_out, phi_in, h_in, Bbar_prev, x_prev); ``grads`` may
    supply preallocated output tensors under those names.  Raw B, C: [b, L, G, R, N]; their
    gradients have the same layout (summed over each group's heads)."""
    lib = load()
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[-1]
    dev, io = x.device, x.dtype
    f32 = torch.float32
    _tensor(B, "B", (b, L, G, R, N), io, dev)
    _tensor(C, "C", (b, L, G, R, N), io, dev)
    _tensor(dt, "dt", (b, L, H), io, dev)
    _tensor(theta, "theta", (b, L, H, N // 2), io, dev)
    _tensor(lam, "lam", (b, L, H), io, dev)
    _tensor(A, "A", (H,), f32, dev)
    _tensor(normw_B, "normw_B", (H, N), f32, dev)
    _tensor(normw_C, "normw_C", (H, N), f32, dev)
    _tensor(bias_B, "bias_B", (H, R, N), f32, dev)
    _tensor(bias_C, "bias_C", (H, R, N), f32, dev)
    _tensor(w_out, "w_out", (H, R, P), f32, dev)
    _tensor(phi_in, "phi_in", (b, H, N // 2), f32, dev)
    _tensor(h_in, "h_in", (b, H, N, P), f32, dev)
    _tensor(Bbar_prev, "Bbar_prev", (b, H, R, N), io, dev)
    _tensor(x_prev, "x_prev", (b, H, R, P), io, dev)
    yshape = (b, L, H, P) if w_out is not None else (b, L, H, R, P)
    _tensor(dy, "dy", yshape, io, dev)
    _tensor(dh_out, "dh_out", (b, H, N, P), f32, dev)
    _tensor(dphi_out, "dphi_out", (b, H, N // 2), f32, dev)
    carry = Bbar_prev is not None and x_prev is not None
    spec = {"x": ((b, L, H, R, P), io), "B": ((b, L, G, R, N), io), "C": ((b, L, G, R, N), io),
            "dt": ((b, L, H), io), "theta": ((b, L, H, N // 2), io), "A": ((H,), f32),
            "lam": ((b, L, H), io), "normw_B": ((H, N), f32), "normw_C": ((H, N), f32),
            "bias_B": ((H, R, N), f32), "bias_C": ((H, R, N), f32), "phi_in": ((b, H, N // 2), f32),
            "h_in": ((b, H, N, P), f32)}
    if w_out is not None:
        spec["w_out"] = ((H, R, P), f32)
    if carry:
        spec["Bbar_prev"] = ((b, H, R, N), io)
        spec["x_prev"] = ((b, H, R, P), io)
    grads = dict(grads or {})
    for k, (shape, dtype) in spec.items():
        if grads.get(k) is None:
            grads[k] = torch.empty(shape, dtype=dtype, device=dev)
        _tensor(grads[k], "grad " + k, shape, dtype, dev)
    grads.setdefault("w_out", None)
    grads.setdefault("Bbar_prev", None)
    grads.setdefault("x_prev", None)
    dims = make_dims(b, L, H, P, N, R, 0, _io_code(io), bcnorm, eps, _groups(H, G))
    need = layer_backward_workspace_bytes(dims)
    if need == 0:
        raise M3Error(M3_E_UNSUPPORTED, "no backward kernel for N=%d P=%d R=%d" % (N, P, R))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    g = grads
    _check(lib.m3_layer_backward(
        ctypes.byref(dims), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(theta), _ptr(normw_B),
        _ptr(normw_C), _ptr(bias_B), _ptr(bias_C), _ptr(A), _ptr(lam), _ptr(w_out), _ptr(phi_in),
        _ptr(h_in), _ptr(Bbar_prev), _ptr(x_prev), _ptr(dy), _ptr(dh_out), _ptr(dphi_out),
        _ptr(g["x"]), _ptr(g["B"]), _ptr(g["C"]), _ptr(g["dt"]), _ptr(g["theta"]), _ptr(g["A"]),
        _ptr(g["lam"]), _ptr(g["normw_B"]), _ptr(g["normw_C"]), _ptr(g["bias_B"]),
        _ptr(g["bias_C"]), _ptr(g["w_out"]), _ptr(g["phi_in"]), _ptr(g["h_in"]),
        _ptr(g["Bbar_prev"]), _ptr(g["x_prev"]), _ptr(workspace), ws_bytes, _stream(stream)))
    return grads
