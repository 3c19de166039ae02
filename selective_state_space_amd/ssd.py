"""Python binding of libssd.so (ctypes).

Argument marshalling only: shapes and dtypes are checked, tensors made
contiguous, output and workspace memory allocated with torch on the input's
device, and the C entry points of ``include/ssd.h`` called with raw device
pointers and torch's current stream.  Every step of the computation runs in
the HIP kernels of libssd.so; if the library is missing this module raises,
it never falls back to another implementation.

The functions carry the C names:

* :func:`ssd_chunked_fwd` -- chunked forward, with the layer options (dt bias,
  softplus, z gate, y in the io dtype) when given;
* :func:`ssd_chunked_fwd_noalloc` -- the same on the library's static
  workspace (no allocation in the library);
* :func:`ssd_chunk_cumsum`, :func:`ssd_chunk_state`, :func:`ssd_state_passing`,
  :func:`ssd_state_fwd`, :func:`ssd_chunk_scan` -- the stages one at a time,
  on a shared workspace;
* :func:`ssd_decode_step` -- one recurrent token, state updated in place;
* :func:`ssd_decode_multi` -- K tokens per sequence, with snapshots and
  draft-tree parents;
* :func:`ssd_decode_step_lp` -- the decode step on a 16-bit state;
* :func:`ssd_chunked_bwd` -- every gradient of the chunked forward;
* :func:`ssd_chunked_fwd_workspace_size`, :func:`ssd_chunked_fwd_workspace_layout`,
  :func:`ssd_chunked_bwd_workspace_size`, :func:`fwd_path` and
  :func:`set_path_override` (which path the forward takes, and a switch for
  tests).
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssd.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ssd.h")

SSD_F32, SSD_BF16 = 0, 1
STATUS = {0: "SSD_OK", -1: "SSD_ERR_NULL", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_UNSUPPORTED",
          -4: "SSD_ERR_ALIGN", -5: "SSD_ERR_WORKSPACE", -6: "SSD_ERR_HIP"}


class SSDError(RuntimeError):
    """A libssd.so entry point returned a non-zero ssd_status."""

    def __init__(self, fn: str, status: int, detail: str):
        super().__init__("%s -> %s (%d): %s" % (fn, STATUS.get(status, "?"), status, detail))
        self.status = status
        self.detail = detail


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32)]


class StateFormat(ctypes.Structure):
    """ssd_state_format."""
    _fields_ = [("dtype", ctypes.c_int32), ("philox_rounds", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("scale", ctypes.c_void_p)]


STATE_DTYPES = {"f32": (0, torch.float32), "f16": (1, torch.float16), "bf16": (2, torch.bfloat16),
                "int16": (3, torch.int16)}


class LayerOpts(ctypes.Structure):
    """ssd_layer_opts: dt_bias [H] f32 (or NULL), dt_softplus, y_io_dtype, z (or NULL)."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("y_io_dtype", ctypes.c_int32), ("z", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libssd.so (built in-tree by ``python -m selective_state_space_amd.build``)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libssd.so is not built (%s); run `python -m "
                           "selective_state_space_amd.build` -- there is no fallback" % path)
    lib = ctypes.CDLL(path)
    vp, i64, sz, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.POINTER(Dims)
    st = ctypes.c_int
    sig = {
        "ssd_chunked_fwd": ([vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, dp, vp, sz, vp], st),
        "ssd_chunked_fwd_workspace_size": ([dp, i64], sz),
        "ssd_chunked_fwd_workspace_layout": ([dp, i64, ctypes.POINTER(ctypes.c_size_t)], st),
        "ssd_chunk_cumsum": ([vp, vp, i64, dp, vp, sz, vp], st),
        "ssd_chunk_state": ([vp, vp, i64, dp, vp, sz, vp], st),
        "ssd_state_passing": ([vp, vp, i64, dp, vp, sz, vp], st),
        "ssd_chunk_scan": ([vp, vp, vp, vp, vp, i64, dp, vp, sz, vp], st),
        "ssd_state_fwd": ([vp, vp, vp, vp, i64, dp, vp, sz, vp], st),
        "ssd_chunked_fwd_opts": ([vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                  ctypes.POINTER(LayerOpts), dp, vp, sz, vp], st),
        "ssd_decode_step_opts": ([vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(LayerOpts), dp,
                                  vp], st),
        "ssd_chunked_fwd_path": ([dp, i64, ctypes.POINTER(ctypes.c_int)], st),
        "ssd_set_path_override": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], st),
        "ssd_chunked_fwd_noalloc": ([vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                     ctypes.POINTER(LayerOpts), dp, vp], st),
        "ssd_decode_step": ([vp, vp, vp, vp, vp, vp, vp, vp, dp, vp], st),
        "ssd_decode_multi": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32,
                              ctypes.POINTER(LayerOpts), dp, vp], st),
        "ssd_chunked_bwd_workspace_size": ([dp, i64], sz),
        "ssd_chunked_bwd": ([vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                             vp, dp, vp, sz, vp], st),
        "ssd_decode_step_lp": ([vp, ctypes.POINTER(StateFormat), vp, vp, vp, vp, vp, vp, vp,
                                ctypes.POINTER(LayerOpts), dp, vp], st),
        "ssd_status_string": ([st], ctypes.c_char_p),
        "ssd_last_error_detail": ([], ctypes.c_char_p),
        "ssd_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions ``include/ssd.h`` declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def _check(fn: str, status: int):
    if status != 0:
        detail = load_library().ssd_last_error_detail().decode()
        raise SSDError(fn, status, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return SSD_F32
    if dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError("x, B, C must be float32 or bfloat16, got %s" % dtype)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t.contiguous()


def _need_out(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> torch.Tensor:
    """An output the library writes into: a contiguous copy would lose the result."""
    if isinstance(t, torch.Tensor) and not t.is_contiguous():
        raise ValueError("%s must be contiguous (the library writes into it)" % name)
    return _need(t, name, dtype, shape, device)


def fwd_dims(x: torch.Tensor, B: torch.Tensor) -> Dims:
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return Dims(Bt, T, H, P, N, G, _io_code(x.dtype))


def ssd_chunked_fwd_workspace_size(dims: Dims, chunk_size: int) -> int:
    return int(load_library().ssd_chunked_fwd_workspace_size(ctypes.byref(dims), chunk_size))


def ssd_chunked_fwd_workspace_layout(dims: Dims, chunk_size: int) -> Tuple[int, int, int, int]:
    off = (ctypes.c_size_t * 4)()
    _check("ssd_chunked_fwd_workspace_layout",
           load_library().ssd_chunked_fwd_workspace_layout(ctypes.byref(dims), chunk_size, off))
    return tuple(int(v) for v in off)


class FwdArgs:
    """Checked, contiguous arguments of one chunked forward (shared by the stage calls)."""

    def __init__(self, x, dt, A, B, C, D, chunk_size, init_state=None, y=None,
                 final_state=None, want_final=True, workspace=None, dt_bias=None,
                 dt_softplus=False, z=None, y_io_dtype=False):
        if x.dim() != 4 or B.dim() != 4:
            raise ValueError("x must be [Bt,T,H,P] and B, C [Bt,T,G,N]")
        dev = x.device
        if dev.type != "cuda":
            raise ValueError("tensors must live on a GPU device, got %s" % dev)
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        io = x.dtype
        self.x = x.contiguous()
        self.dt = _need(dt, "dt", torch.float32, (Bt, T, H), dev)
        self.A = _need(A, "A", torch.float32, (H,), dev)
        self.B = _need(B, "B", io, (Bt, T, G, N), dev)
        self.C = _need(C, "C", io, (Bt, T, G, N), dev)
        self.D = _need(D, "D", torch.float32, (H,), dev)
        self.init = None if init_state is None else _need(init_state, "init_state", torch.float32,
                                                         (Bt, H, P, N), dev)
        self.y_io_dtype = bool(y_io_dtype)
        ydt = io if self.y_io_dtype else torch.float32
        self.y = (torch.empty((Bt, T, H, P), dtype=ydt, device=dev) if y is None
                  else _need_out(y, "y", ydt, (Bt, T, H, P), dev))
        if final_state is not None:
            self.final = _need_out(final_state, "final_state", torch.float32, (Bt, H, P, N), dev)
        elif want_final:
            self.final = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
        else:
            self.final = None
        self.L = int(chunk_size)
        self.dt_bias = None if dt_bias is None else _need(dt_bias, "dt_bias", torch.float32,
                                                          (H,), dev)
        self.z = None if z is None else _need(z, "z", io, (Bt, T, H, P), dev)
        self.dt_softplus = bool(dt_softplus)
        self.dims = fwd_dims(self.x, self.B)
        need = ssd_chunked_fwd_workspace_size(self.dims, self.L)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.ws = workspace
        self.device = dev


def _layer_opts(dt_bias, dt_softplus, z, y_io_dtype=False):
    if dt_bias is None and not dt_softplus and z is None and not y_io_dtype:
        return None
    return LayerOpts(_ptr(dt_bias), int(bool(dt_softplus)), int(bool(y_io_dtype)), _ptr(z))


def ssd_chunked_fwd(x, dt=None, A=None, B=None, C=None, D=None, chunk_size=None,
                    init_state=None, y=None, final_state=None, want_final: bool = True,
                    workspace=None, dt_bias=None, dt_softplus: bool = False, z=None,
                    y_io_dtype: bool = False):
    """Chunked forward.  Returns (y, final_state or None).

    x [Bt,T,H,P] (float32 or bfloat16), dt [Bt,T,H] f32, A/D [H] f32,
    B/C [Bt,T,G,N] (x's dtype), init_state [Bt,H,P,N] f32 or None.  y is
    [Bt,T,H,P], float32 whatever the input dtype unless ``y_io_dtype``.  ``y``,
    ``final_state`` and ``workspace`` may be passed in to avoid allocation;
    ``final_state`` may be the same tensor as ``init_state``.  ``x`` may
    instead be a prepared FwdArgs (then the other arguments are ignored).
    ``dt_bias`` [H] f32, ``dt_softplus`` and the gate ``z`` (x's shape and
    dtype) are the optional layer interface (ssd_layer_opts); ``y_io_dtype``
    stores y in x's dtype instead of float32.
    """
    if isinstance(x, FwdArgs):
        a = x
    else:
        if any(v is None for v in (dt, A, B, C, D, chunk_size)):
            raise ValueError("ssd_chunked_fwd needs x, dt, A, B, C, D and chunk_size")
        a = FwdArgs(x, dt, A, B, C, D, chunk_size, init_state, y, final_state, want_final,
                    workspace, dt_bias, dt_softplus, z, y_io_dtype)
    lib = load_library()
    opts = _layer_opts(a.dt_bias, a.dt_softplus, a.z, a.y_io_dtype)
    if opts is None:
        st = lib.ssd_chunked_fwd(_ptr(a.x), _ptr(a.dt), _ptr(a.A), _ptr(a.B), _ptr(a.C),
                                 _ptr(a.D), a.L, _ptr(a.init), _ptr(a.y), _ptr(a.final),
                                 ctypes.byref(a.dims), _ptr(a.ws), a.ws.numel(),
                                 _stream(a.device))
        _check("ssd_chunked_fwd", st)
    else:
        st = lib.ssd_chunked_fwd_opts(_ptr(a.x), _ptr(a.dt), _ptr(a.A), _ptr(a.B), _ptr(a.C),
                                      _ptr(a.D), a.L, _ptr(a.init), _ptr(a.y), _ptr(a.final),
                                      ctypes.byref(opts), ctypes.byref(a.dims), _ptr(a.ws),
                                      a.ws.numel(), _stream(a.device))
        _check("ssd_chunked_fwd_opts", st)
    return a.y, a.final


NOALLOC_SCRATCH_BYTES = 64 << 20   # SSD_NOALLOC_SCRATCH_BYTES


def ssd_chunked_fwd_noalloc(x, dt, A, B, C, D, chunk_size, init_state=None, y=None,
                            final_state=None, want_final: bool = True, dt_bias=None,
                            dt_softplus: bool = False, z=None, y_io_dtype: bool = False):
    """ssd_chunked_fwd on the library's static scratch (no workspace is
    allocated or passed).  Returns (y, final_state or None).  Shapes whose
    workspace exceeds NOALLOC_SCRATCH_BYTES raise SSDError (SSD_ERR_WORKSPACE)."""
    a = FwdArgs(x, dt, A, B, C, D, chunk_size, init_state, y, final_state, want_final,
                torch.empty(0, dtype=torch.uint8, device=x.device), dt_bias, dt_softplus, z,
                y_io_dtype)
    opts = _layer_opts(a.dt_bias, a.dt_softplus, a.z, a.y_io_dtype)
    st = load_library().ssd_chunked_fwd_noalloc(
        _ptr(a.x), _ptr(a.dt), _ptr(a.A), _ptr(a.B), _ptr(a.C), _ptr(a.D), a.L, _ptr(a.init),
        _ptr(a.y), _ptr(a.final), None if opts is None else ctypes.byref(opts),
        ctypes.byref(a.dims), _stream(a.device))
    _check("ssd_chunked_fwd_noalloc", st)
    return a.y, a.final


def ssd_chunk_cumsum(a: FwdArgs):
    lib = load_library()
    _check("ssd_chunk_cumsum", lib.ssd_chunk_cumsum(_ptr(a.dt), _ptr(a.A), a.L,
                                                    ctypes.byref(a.dims), _ptr(a.ws),
                                                    a.ws.numel(), _stream(a.device)))


def ssd_chunk_state(a: FwdArgs):
    lib = load_library()
    _check("ssd_chunk_state", lib.ssd_chunk_state(_ptr(a.x), _ptr(a.B), a.L, ctypes.byref(a.dims),
                                                  _ptr(a.ws), a.ws.numel(), _stream(a.device)))


def ssd_state_passing(a: FwdArgs):
    lib = load_library()
    _check("ssd_state_passing", lib.ssd_state_passing(_ptr(a.init), _ptr(a.final), a.L,
                                                      ctypes.byref(a.dims), _ptr(a.ws),
                                                      a.ws.numel(), _stream(a.device)))


def ssd_state_fwd(a: FwdArgs):
    """chunk_state + state_passing in one pass (bf16): h_prev and final_state."""
    lib = load_library()
    _check("ssd_state_fwd", lib.ssd_state_fwd(_ptr(a.x), _ptr(a.B), _ptr(a.init), _ptr(a.final),
                                              a.L, ctypes.byref(a.dims), _ptr(a.ws),
                                              a.ws.numel(), _stream(a.device)))


PATH_FOUR_STAGE, PATH_STATE_FWD, PATH_FUSED = 0, 1, 2   # ssd_fwd_path


def fwd_path(dims: Dims, chunk_size: int) -> int:
    """The ssd_fwd_path ssd_chunked_fwd takes for this shape."""
    out = ctypes.c_int(-1)
    _check("ssd_chunked_fwd_path", load_library().ssd_chunked_fwd_path(
        ctypes.byref(dims), chunk_size, ctypes.byref(out)))
    return out.value


def set_path_override(fwd: int = -1, state_rows: int = 0, adj_rows: int = 0):
    """Test hook (ssd_set_path_override): force a forward path and row splits
    for later calls in this process; (-1, 0, 0) restores the default."""
    _check("ssd_set_path_override",
           load_library().ssd_set_path_override(int(fwd), int(state_rows), int(adj_rows)))


def ssd_chunk_scan(a: FwdArgs):
    """The chunk_scan stage (no layer options): writes y in float32."""
    if a.y.dtype != torch.float32:
        raise ValueError("the stage call ssd_chunk_scan writes y in float32; these arguments "
                         "hold a %s y (y_io_dtype): use ssd_chunked_fwd" % a.y.dtype)
    lib = load_library()
    _check("ssd_chunk_scan", lib.ssd_chunk_scan(_ptr(a.x), _ptr(a.B), _ptr(a.C), _ptr(a.D),
                                                _ptr(a.y), a.L, ctypes.byref(a.dims), _ptr(a.ws),
                                                a.ws.numel(), _stream(a.device)))


def workspace_views(a: FwdArgs):
    """Views of the intermediates a forward left in ``a.ws``: G, DT, S, h_prev."""
    Bt, T, H, P = a.x.shape
    N = a.B.shape[3]
    nc = -(-T // a.L)
    off = ssd_chunked_fwd_workspace_layout(a.dims, a.L)

    def view(o, n, dtype, shape):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return a.ws[o:o + nbytes].view(dtype).view(shape)

    units = Bt * H * nc
    return {
        "G": view(off[0], units * a.L, torch.float32, (Bt, H, nc, a.L)),
        "DT": view(off[1], units * a.L, torch.float32, (Bt, H, nc, a.L)),
        "S": view(off[2], units * P * N, torch.float32, (Bt, H, nc, P, N)),
        "h_prev": view(off[3], units * P * N, a.x.dtype, (Bt, H, nc, P, N)),
    }


def ssd_decode_step(state, x_t, dt_t, B_t, C_t, A, D, y_t=None, dt_bias=None,
                    dt_softplus: bool = False, z_t=None, y_io_dtype: bool = False):
    """One decode step; ``state`` [Bt,H,P,N] f32 is updated in place.  Returns y_t [Bt,H,P] f32.

    ``dt_bias`` [H], ``dt_softplus`` and the gate ``z_t`` [Bt,H,P] (x_t's dtype)
    are the optional layer interface (ssd_layer_opts); ``y_io_dtype`` stores
    y_t in x_t's dtype instead of float32.
    """
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device, got %s" % dev)
    if not state.is_contiguous() or state.dtype != torch.float32 or state.dim() != 4:
        raise ValueError("state must be a contiguous float32 [Bt,H,P,N] tensor (updated in place)")
    Bt, H, P, N = state.shape
    io = x_t.dtype
    G = B_t.shape[1]
    x_t = _need(x_t, "x_t", io, (Bt, H, P), dev)
    dt_t = _need(dt_t, "dt_t", torch.float32, (Bt, H), dev)
    B_t = _need(B_t, "B_t", io, (Bt, G, N), dev)
    C_t = _need(C_t, "C_t", io, (Bt, G, N), dev)
    A = _need(A, "A", torch.float32, (H,), dev)
    D = _need(D, "D", torch.float32, (H,), dev)
    ydt = io if y_io_dtype else torch.float32
    y_t = (torch.empty((Bt, H, P), dtype=ydt, device=dev) if y_t is None
           else _need_out(y_t, "y_t", ydt, (Bt, H, P), dev))
    dims = Dims(Bt, 1, H, P, N, G, _io_code(io))
    if dt_bias is not None:
        dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    if z_t is not None:
        z_t = _need(z_t, "z_t", io, (Bt, H, P), dev)
    lib = load_library()
    opts = _layer_opts(dt_bias, dt_softplus, z_t, y_io_dtype)
    if opts is None:
        _check("ssd_decode_step", lib.ssd_decode_step(_ptr(state), _ptr(x_t), _ptr(dt_t),
                                                      _ptr(B_t), _ptr(C_t), _ptr(A), _ptr(D),
                                                      _ptr(y_t), ctypes.byref(dims),
                                                      _stream(dev)))
    else:
        _check("ssd_decode_step_opts", lib.ssd_decode_step_opts(
            _ptr(state), _ptr(x_t), _ptr(dt_t), _ptr(B_t), _ptr(C_t), _ptr(A), _ptr(D),
            _ptr(y_t), ctypes.byref(opts), ctypes.byref(dims), _stream(dev)))
    return y_t


DECODE_NO_STATE_UPDATE = 1   # SSD_DECODE_NO_STATE_UPDATE


def ssd_decode_multi(state, x, dt, B, C, A, D, y=None, snapshots=None, parent=None,
                     update_state: bool = True, dt_bias=None, dt_softplus: bool = False, z=None,
                     y_io_dtype: bool = False):
    """K decode steps per sequence (speculative decoding); returns (y, snapshots).

    state [Bt,H,P,N] f32 (updated in place unless ``update_state`` is False),
    x [Bt,K,H,P], dt [Bt,K,H] f32, B/C [Bt,K,G,N] (x's dtype), A/D [H] f32.
    ``snapshots``: None (not written), True (allocated here) or a float32
    [Bt,K,H,P,N] tensor that receives the state after every step.  ``parent``
    [Bt,K] int32: step k restarts from the snapshot of step parent[b,k] when
    0 <= parent[b,k] < k (needs snapshots).  y [Bt,K,H,P] f32.
    """
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device, got %s" % dev)
    if not state.is_contiguous() or state.dtype != torch.float32 or state.dim() != 4:
        raise ValueError("state must be a contiguous float32 [Bt,H,P,N] tensor")
    Bt, H, P, N = state.shape
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [Bt,K,H,P] and B, C [Bt,K,G,N]")
    io = x.dtype
    K, G = x.shape[1], B.shape[2]
    x = _need(x, "x", io, (Bt, K, H, P), dev)
    dt = _need(dt, "dt", torch.float32, (Bt, K, H), dev)
    B = _need(B, "B", io, (Bt, K, G, N), dev)
    C = _need(C, "C", io, (Bt, K, G, N), dev)
    A = _need(A, "A", torch.float32, (H,), dev)
    D = _need(D, "D", torch.float32, (H,), dev)
    ydt = io if y_io_dtype else torch.float32
    y = (torch.empty((Bt, K, H, P), dtype=ydt, device=dev) if y is None
         else _need_out(y, "y", ydt, (Bt, K, H, P), dev))
    if snapshots is True:
        snapshots = torch.empty((Bt, K, H, P, N), dtype=torch.float32, device=dev)
    elif snapshots is not None:
        snapshots = _need_out(snapshots, "snapshots", torch.float32, (Bt, K, H, P, N), dev)
    if parent is not None:
        parent = _need(parent, "parent", torch.int32, (Bt, K), dev)
    if dt_bias is not None:
        dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    if z is not None:
        z = _need(z, "z", io, (Bt, K, H, P), dev)
    opts = _layer_opts(dt_bias, dt_softplus, z, y_io_dtype)
    dims = Dims(Bt, K, H, P, N, G, _io_code(io))
    flags = 0 if update_state else DECODE_NO_STATE_UPDATE
    _check("ssd_decode_multi", load_library().ssd_decode_multi(
        _ptr(state), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(y),
        _ptr(snapshots), _ptr(parent), flags, None if opts is None else ctypes.byref(opts),
        ctypes.byref(dims), _stream(dev)))
    return y, snapshots


def ssd_decode_step_lp(state, x_t, dt_t, B_t, C_t, A, D, fmt: str, scale=None,
                       philox_rounds: int = 0, seed: int = 0, y_t=None, dt_bias=None,
                       dt_softplus: bool = False, z_t=None, y_io_dtype: bool = False):
    """One decode step on a 16-bit state (``fmt`` "f16", "bf16" or "int16"; "f32"
    is the plain step), updated in place.  state [Bt,H,P,N] of fp16 / bf16 /
    int16; ``scale`` [Bt,H,P] f32 decode scales (int16 only, updated in place);
    ``philox_rounds`` > 0 (10 is standard) and ``seed`` select fp16
    stochastic rounding.  Returns y_t
    [Bt,H,P] f32."""
    if fmt not in STATE_DTYPES:
        raise ValueError("fmt must be one of %s" % sorted(STATE_DTYPES))
    code, sdt = STATE_DTYPES[fmt]
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device, got %s" % dev)
    if not state.is_contiguous() or state.dtype != sdt or state.dim() != 4:
        raise ValueError("state must be a contiguous %s [Bt,H,P,N] tensor" % sdt)
    Bt, H, P, N = state.shape
    io = x_t.dtype
    G = B_t.shape[1]
    x_t = _need(x_t, "x_t", io, (Bt, H, P), dev)
    dt_t = _need(dt_t, "dt_t", torch.float32, (Bt, H), dev)
    B_t = _need(B_t, "B_t", io, (Bt, G, N), dev)
    C_t = _need(C_t, "C_t", io, (Bt, G, N), dev)
    A = _need(A, "A", torch.float32, (H,), dev)
    D = _need(D, "D", torch.float32, (H,), dev)
    ydt = io if y_io_dtype else torch.float32
    y_t = (torch.empty((Bt, H, P), dtype=ydt, device=dev) if y_t is None
           else _need_out(y_t, "y_t", ydt, (Bt, H, P), dev))
    if scale is not None:
        scale = _need_out(scale, "scale", torch.float32, (Bt, H, P), dev)
    if dt_bias is not None:
        dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    if z_t is not None:
        z_t = _need(z_t, "z_t", io, (Bt, H, P), dev)
    f = StateFormat(code, int(philox_rounds), int(seed) & 0xFFFFFFFFFFFFFFFF,
                    None if scale is None else scale.data_ptr())
    opts = _layer_opts(dt_bias, dt_softplus, z_t, y_io_dtype)
    dims = Dims(Bt, 1, H, P, N, G, _io_code(io))
    _check("ssd_decode_step_lp", load_library().ssd_decode_step_lp(
        _ptr(state), ctypes.byref(f), _ptr(x_t), _ptr(dt_t), _ptr(B_t), _ptr(C_t), _ptr(A),
        _ptr(D), _ptr(y_t), None if opts is None else ctypes.byref(opts), ctypes.byref(dims),
        _stream(dev)))
    return y_t


def ssd_chunked_bwd_workspace_size(dims: Dims, chunk_size: int) -> int:
    return int(load_library().ssd_chunked_bwd_workspace_size(ctypes.byref(dims), chunk_size))


def ssd_chunked_bwd(x, dt, A, B, C, D, chunk_size, dy, init_state=None, dfinal=None,
                    want_dinit: bool = True, workspace=None):
    """Backward of ssd_chunked_fwd (no layer options).  Returns a dict of float32
    gradients: dx [Bt,T,H,P], ddt [Bt,T,H], dA [H], dB and dC [Bt,T,G,N], dD [H],
    dinit [Bt,H,P,N] (None unless ``want_dinit``).  dy [Bt,T,H,P] f32; dfinal
    [Bt,H,P,N] f32 or None."""
    a = FwdArgs(x, dt, A, B, C, D, chunk_size, init_state, want_final=False,
                workspace=torch.empty(256, dtype=torch.uint8, device=x.device))
    Bt, T, H, P = a.x.shape
    G, N = a.B.shape[2], a.B.shape[3]
    dev = a.device
    dy = _need(dy, "dy", torch.float32, (Bt, T, H, P), dev)
    if dfinal is not None:
        dfinal = _need(dfinal, "dfinal", torch.float32, (Bt, H, P, N), dev)
    need = ssd_chunked_bwd_workspace_size(a.dims, a.L)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty((Bt, T, H, P), **f32), ddt=torch.empty((Bt, T, H), **f32),
               dA=torch.empty((H,), **f32), dB=torch.empty((Bt, T, G, N), **f32),
               dC=torch.empty((Bt, T, G, N), **f32), dD=torch.empty((H,), **f32),
               dinit=torch.empty((Bt, H, P, N), **f32) if want_dinit else None)
    _check("ssd_chunked_bwd", load_library().ssd_chunked_bwd(
        _ptr(a.x), _ptr(a.dt), _ptr(a.A), _ptr(a.B), _ptr(a.C), _ptr(a.D), a.L, _ptr(a.init),
        _ptr(dy), _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]),
        ctypes.byref(a.dims), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out
