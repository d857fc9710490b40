"""Python binding of libssd, the MI355X (gfx950) chunked SSD forward.

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libssd.so``; torch supplies device memory and the stream.  There is no fallback: if the
library is not built, or a tensor is not on a GPU, the call raises.

The functions carry the names of the C entry points declared in ``include/ssd.h``:
  ssd_forward_workspace_bytes(dims, chunk) -> int
  ssd_forward(x, log_a, B, C, D=None, chunk=..., init_state=None, y=None,
              final_state=None, workspace=None, stream=None) -> (y, final_state)
  ssd_forward_profiled(..., events=(hipEvent_t handles)) -> (y, final_state, n_launches)
  ssd_step(state, x_t, log_a_t, B_t, C_t, D=None, y_t=None, stream=None) -> y_t
  ssd_forward_dt_workspace_bytes(dims, chunk, scale_input) -> int
  ssd_forward_dt(x, dt, A_log, B, C, D=None, dt_bias=None, scale_input=True, chunk=..., ...)
  ssd_forward_dt_profiled(..., events=(hipEvent_t handles)) -> (y, final_state, n_launches)
  ssd_step_dt(state, x_t, dt_t, A_log, B_t, C_t, D=None, dt_bias=None, scale_input=True, ...)
  ssd_backward_workspace_bytes(dims) -> int
  ssd_backward(x, log_a, B, C, dy, D=None, init_state=None, dfinal=None, ...) -> dict of gradients
  ssd_backward_profiled(..., events=(hipEvent_t handles)) -> (gradients, n_launches)
  ssd_backward_dt_workspace_bytes(dims, scale_input) -> int
  ssd_backward_dt(x, dt, A_log, B, C, dy, D=None, dt_bias=None, scale_input=True, ...) -> dict
  ssd_noalloc_scratch_bytes() -> int
  ssd_forward_noalloc(x, log_a, B, C, D=None, chunk=..., init_state=None, y=None,
                      final_state=None, stream=None) -> (y, final_state)
  ssd_strerror(code) -> str
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["SSDError", "Dims", "library_path", "load_library", "dims_for",
           "ssd_forward_workspace_bytes", "ssd_forward", "ssd_forward_profiled", "ssd_step",
           "ssd_forward_dt_workspace_bytes", "ssd_forward_dt", "ssd_forward_dt_profiled",
           "ssd_step_dt", "ssd_backward_workspace_bytes", "ssd_backward", "ssd_backward_profiled",
           "ssd_backward_dt_workspace_bytes", "ssd_backward_dt",
           "ssd_forward_noalloc", "ssd_noalloc_scratch_bytes", "ssd_strerror",
           "SSD_F32", "SSD_BF16", "SSD_DECAY_SCALAR", "SSD_DECAY_DIAG"]

SSD_F32, SSD_BF16 = 0, 1
SSD_DECAY_SCALAR, SSD_DECAY_DIAG = 0, 1
SSD_OK, SSD_ERR_INVALID, SSD_ERR_UNSUPPORTED, SSD_ERR_ALIGN, SSD_ERR_HIP, SSD_ERR_SCRATCH = 0, -1, -2, -3, -4, -5

_HERE = os.path.dirname(os.path.abspath(__file__))
_DTYPE_CODE = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}


class SSDError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, ssd_strerror(code), code))


class Dims(ctypes.Structure):
    """Mirror of ``ssd_dims``."""
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("decay", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("SSD_LIBRARY", os.path.join(_HERE, "libssd.so"))


_LIB = None


def load_library():
    """Load libssd.so (built in-tree by ``ssd_chunked_scan_02_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("libssd.so is not built (%s); run "
                               "`python -m ssd_chunked_scan_02_amd.build` first" % path)
        lib = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        dp = ctypes.POINTER(Dims)
        lib.ssd_forward_workspace_bytes.argtypes = [dp, i32]
        lib.ssd_forward_workspace_bytes.restype = sz
        lib.ssd_forward.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward.restype = i32
        lib.ssd_forward_profiled.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp,
                                             ctypes.POINTER(vp), i32, ctypes.POINTER(i32)]
        lib.ssd_forward_profiled.restype = i32
        lib.ssd_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ssd_step.restype = i32
        lib.ssd_forward_dt_workspace_bytes.argtypes = [dp, i32, i32]
        lib.ssd_forward_dt_workspace_bytes.restype = sz
        dt_args = [dp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        lib.ssd_forward_dt.argtypes = dt_args
        lib.ssd_forward_dt.restype = i32
        lib.ssd_forward_dt_profiled.argtypes = dt_args + [ctypes.POINTER(vp), i32, ctypes.POINTER(i32)]
        lib.ssd_forward_dt_profiled.restype = i32
        lib.ssd_step_dt.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
        lib.ssd_step_dt.restype = i32
        lib.ssd_backward_workspace_bytes.argtypes = [dp]
        lib.ssd_backward_workspace_bytes.restype = sz
        lib.ssd_backward.argtypes = [dp] + [vp] * 15 + [sz, vp]
        lib.ssd_backward.restype = i32
        lib.ssd_backward_profiled.argtypes = [dp] + [vp] * 15 + [sz, vp, ctypes.POINTER(vp), i32,
                                                                 ctypes.POINTER(i32)]
        lib.ssd_backward_profiled.restype = i32
        lib.ssd_backward_dt_workspace_bytes.argtypes = [dp, i32]
        lib.ssd_backward_dt_workspace_bytes.restype = sz
        lib.ssd_backward_dt.argtypes = [dp, vp, vp, vp, vp, i32] + [vp] * 15 + [sz, vp]
        lib.ssd_backward_dt.restype = i32
        lib.ssd_forward_varlen_workspace_bytes.argtypes = [dp, i32]
        lib.ssd_forward_varlen_workspace_bytes.restype = sz
        lib.ssd_forward_varlen.argtypes = [dp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz,
                                           vp, ctypes.POINTER(vp), i32, ctypes.POINTER(i32)]
        lib.ssd_forward_varlen.restype = i32
        lib.ssd_forward_dt_varlen_workspace_bytes.argtypes = [dp, i32, i32]
        lib.ssd_forward_dt_varlen_workspace_bytes.restype = sz
        lib.ssd_forward_dt_varlen.argtypes = [dp, vp, ctypes.c_int64, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp,
                                              vp, vp, sz, vp, ctypes.POINTER(vp), i32, ctypes.POINTER(i32)]
        lib.ssd_forward_dt_varlen.restype = i32
        lib.ssd_backward_varlen_workspace_bytes.argtypes = [dp]
        lib.ssd_backward_varlen_workspace_bytes.restype = sz
        lib.ssd_backward_varlen.argtypes = [dp, vp, ctypes.c_int64] + [vp] * 15 + [sz, vp, ctypes.POINTER(vp), i32,
                                                                             ctypes.POINTER(i32)]
        lib.ssd_backward_varlen.restype = i32
        lib.ssd_backward_dt_varlen_workspace_bytes.argtypes = [dp, i32]
        lib.ssd_backward_dt_varlen_workspace_bytes.restype = sz
        lib.ssd_backward_dt_varlen.argtypes = [dp, vp, ctypes.c_int64, vp, vp, vp, vp, i32] + [vp] * 15 + [sz, vp]
        lib.ssd_backward_dt_varlen.restype = i32
        lib.ssd_noalloc_scratch_bytes.argtypes = []
        lib.ssd_noalloc_scratch_bytes.restype = sz
        lib.ssd_forward_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
        lib.ssd_forward_noalloc.restype = i32
        lib.ssd_strerror.argtypes = [i32]
        lib.ssd_strerror.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def ssd_strerror(code: int) -> str:
    return load_library().ssd_strerror(int(code)).decode()


def dims_for(x: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor) -> Dims:
    """ssd_dims of a forward call: x [B,T,H,P], log_a [B,T,H] or [B,T,H,N], B [B,T,G,N]."""
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [B,T,H,P] and B [B,T,G,N]")
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    decay = SSD_DECAY_DIAG if log_a.dim() == 4 else SSD_DECAY_SCALAR
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    return Dims(bsz, T, H, G, P, N, _DTYPE_CODE[x.dtype], decay)


def ssd_forward_workspace_bytes(dims: Dims, chunk: int) -> int:
    return int(load_library().ssd_forward_workspace_bytes(ctypes.byref(dims), int(chunk)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream, *tensors):
    """Mark the tensors a call reads or writes as used on the caller's launch stream when that is
    not torch's current stream: the caching allocator then waits for the kernels on that stream
    before it hands their memory to another allocation (the wrapper's own workspace is freed on
    return, and outputs may be dropped by the caller on another stream)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


SSD_MAX_LAUNCHES = 4


def ssd_forward(x, log_a, B, C, D=None, chunk: int = 64, init_state=None, y=None,
                final_state=None, workspace=None, stream=None):
    """Run ``ssd_forward`` on the GPU.

    ``y`` and the workspace are allocated when not given.  ``final_state`` may be a tensor
    to write, True to allocate one, or None/False to skip it.  Returns (y, final_state).
    """
    return _forward(x, log_a, B, C, D, chunk, init_state, y, final_state, workspace, stream)[:2]


def ssd_forward_profiled(x, log_a, B, C, D=None, chunk: int = 64, init_state=None, y=None,
                         final_state=None, workspace=None, stream=None, events=()):
    """``ssd_forward_profiled``: as ssd_forward; launch k stamps the hipEvent_t handles
    (integers) events[2k] at its start and events[2k+1] at its end.
    Returns (y, final_state, n_launches)."""
    return _forward(x, log_a, B, C, D, chunk, init_state, y, final_state, workspace, stream,
                    events=list(events))


def _forward(x, log_a, B, C, D, chunk, init_state, y, final_state, workspace, stream,
             events=None):
    dims = dims_for(x, log_a, B)
    dev = x.device
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check(x, "x", (bsz, T, H, P), x.dtype, dev)
    la_shape = (bsz, T, H, N) if dims.decay == SSD_DECAY_DIAG else (bsz, T, H)
    _check(log_a, "log_a", la_shape, torch.float32, dev)
    _check(B, "B", (bsz, T, G, N), x.dtype, dev)
    _check(C, "C", (bsz, T, G, N), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (bsz, H, N, P), torch.float32, dev)
    if y is None:
        y = torch.empty((bsz, T, H, P), dtype=x.dtype, device=dev)
    _check(y, "y", (bsz, T, H, P), x.dtype, dev)
    if final_state is True:
        final_state = torch.empty((bsz, H, N, P), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    _check(final_state, "final_state", (bsz, H, N, P), torch.float32, dev)
    lib = load_library()
    need = int(lib.ssd_forward_workspace_bytes(ctypes.byref(dims), int(chunk)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(dims), _ptr(x), _ptr(log_a), _ptr(B), _ptr(C), _ptr(D), int(chunk),
            _ptr(init_state), _ptr(y), _ptr(final_state), _ptr(workspace), ws_bytes,
            _stream_handle(stream, dev))
    _on_stream(stream, y, final_state, workspace)
    if events is None:
        rc = lib.ssd_forward(*args)
        launches = None
    else:
        n = max(len(events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(events) + [None] * (n - len(events))))
        count = ctypes.c_int(0)
        rc = lib.ssd_forward_profiled(*args, arr, n, ctypes.byref(count))
        launches = count.value
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_forward")
    return y, final_state, launches


def ssd_noalloc_scratch_bytes() -> int:
    return int(load_library().ssd_noalloc_scratch_bytes())


def ssd_forward_noalloc(x, log_a, B, C, D=None, chunk: int = 64, init_state=None, y=None, final_state=None,
                        stream=None):
    """Run ``ssd_forward_noalloc``: ssd_forward with its workspace in the library's fixed per-GPU
    scratch array, so the C call allocates nothing (pass ``y`` and ``final_state`` as well for a
    call that allocates nothing at all, e.g. under graph capture).  Raises SSDError with
    SSD_ERR_SCRATCH when the workload's workspace is larger than the array.
    Returns (y, final_state)."""
    dims = dims_for(x, log_a, B)
    dev = x.device
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check(x, "x", (bsz, T, H, P), x.dtype, dev)
    _check(log_a, "log_a", (bsz, T, H, N) if dims.decay == SSD_DECAY_DIAG else (bsz, T, H), torch.float32, dev)
    _check(B, "B", (bsz, T, G, N), x.dtype, dev)
    _check(C, "C", (bsz, T, G, N), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (bsz, H, N, P), torch.float32, dev)
    if y is None:
        y = torch.empty((bsz, T, H, P), dtype=x.dtype, device=dev)
        _on_stream(stream, y)
    _check(y, "y", (bsz, T, H, P), x.dtype, dev)
    if final_state is True:
        final_state = torch.empty((bsz, H, N, P), dtype=torch.float32, device=dev)
        _on_stream(stream, final_state)
    elif final_state is False:
        final_state = None
    _check(final_state, "final_state", (bsz, H, N, P), torch.float32, dev)
    rc = load_library().ssd_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(log_a), _ptr(B), _ptr(C), _ptr(D),
                                            int(chunk), _ptr(init_state), _ptr(y), _ptr(final_state),
                                            _stream_handle(stream, dev))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_forward_noalloc")
    return y, final_state


def varlen_dims(x: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, nseq: int, max_seqlen: int) -> Dims:
    """ssd_dims of a packed variable-length call: x [T,H,P], log_a [T,H] or [T,H,N], B [T,G,N];
    nseq sequences of at most max_seqlen tokens."""
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [T,H,P] and B [T,G,N]")
    _, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    decay = SSD_DECAY_DIAG if log_a.dim() == 3 else SSD_DECAY_SCALAR
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    return Dims(int(nseq), int(max_seqlen), H, G, P, N, _DTYPE_CODE[x.dtype], decay)


def ssd_forward_varlen_workspace_bytes(dims: Dims, chunk: int) -> int:
    return int(load_library().ssd_forward_varlen_workspace_bytes(ctypes.byref(dims), int(chunk)))


def ssd_forward_varlen(x, log_a, B, C, cu_seqlens, max_seqlen: int, D=None, chunk: int = 64, init_state=None,
                       y=None, final_state=None, workspace=None, stream=None, events=None):
    """Run ``ssd_forward_varlen``: a packed batch of len(cu_seqlens) - 1 sequences, sequence i
    being tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1 of x [T,H,P], log_a [T,H] or [T,H,N],
    B, C [T,G,N].  cu_seqlens: int64 tensor on the GPU; max_seqlen: a bound on every length
    (host int).  init_state / final_state [nseq,H,N,P] fp32 as in ssd_forward.  With ``events``
    (hipEvent_t handles) launch k stamps events[2k] and events[2k+1].
    Returns (y, final_state, n_launches or None)."""
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or nseq < 0 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor of nseq + 1 offsets on x's device")
    dims = varlen_dims(x, log_a, B, nseq, max_seqlen)
    _check(x, "x", (T, H, P), x.dtype, dev)
    _check(log_a, "log_a", (T, H, N) if dims.decay == SSD_DECAY_DIAG else (T, H), torch.float32, dev)
    _check(B, "B", (T, G, N), x.dtype, dev)
    _check(C, "C", (T, G, N), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (nseq, H, N, P), torch.float32, dev)
    if y is None:
        y = torch.empty((T, H, P), dtype=x.dtype, device=dev)
    _check(y, "y", (T, H, P), x.dtype, dev)
    if final_state is True:
        final_state = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    _check(final_state, "final_state", (nseq, H, N, P), torch.float32, dev)
    lib = load_library()
    need = int(lib.ssd_forward_varlen_workspace_bytes(ctypes.byref(dims), int(chunk)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr, n, count = None, 0, ctypes.c_int(0)
    if events is not None:
        n = max(len(events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(events) + [None] * (n - len(events))))
    _on_stream(stream, y, final_state, workspace)
    rc = lib.ssd_forward_varlen(ctypes.byref(dims), _ptr(cu_seqlens), int(T), _ptr(x), _ptr(log_a), _ptr(B),
                                _ptr(C), _ptr(D), int(chunk), _ptr(init_state), _ptr(y), _ptr(final_state),
                                _ptr(workspace), ws_bytes, _stream_handle(stream, dev), arr, n,
                                ctypes.byref(count))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_forward_varlen")
    return y, final_state, (count.value if events is not None else None)


def ssd_forward_dt_varlen_workspace_bytes(dims: Dims, chunk: int, scale_input: bool = True) -> int:
    return int(load_library().ssd_forward_dt_varlen_workspace_bytes(ctypes.byref(dims), int(chunk),
                                                                    1 if scale_input else 0))


def ssd_forward_dt_varlen(x, dt, A_log, B, C, cu_seqlens, max_seqlen: int, D=None, dt_bias=None,
                          scale_input: bool = True, chunk: int = 64, init_state=None, y=None, final_state=None,
                          workspace=None, stream=None, events=None):
    """Run ``ssd_forward_dt_varlen``: ssd_forward_varlen with log a = -softplus(dt + dt_bias)
    exp(A_log) and (scale_input) the input scale formed in the kernels.  dt [T,H] fp32; A_log [H]
    or [H,N]; dt_bias [H] or None.  Returns (y, final_state, n_launches or None)."""
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or nseq < 0 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor of nseq + 1 offsets on x's device")
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    decay = SSD_DECAY_DIAG if A_log.dim() == 2 else SSD_DECAY_SCALAR
    dims = Dims(int(nseq), int(max_seqlen), H, G, P, N, _DTYPE_CODE[x.dtype], decay)
    _check(x, "x", (T, H, P), x.dtype, dev)
    _check(dt, "dt", (T, H), torch.float32, dev)
    _check(A_log, "A_log", (H, N) if decay == SSD_DECAY_DIAG else (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B, "B", (T, G, N), x.dtype, dev)
    _check(C, "C", (T, G, N), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (nseq, H, N, P), torch.float32, dev)
    if y is None:
        y = torch.empty((T, H, P), dtype=x.dtype, device=dev)
    _check(y, "y", (T, H, P), x.dtype, dev)
    if final_state is True:
        final_state = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    _check(final_state, "final_state", (nseq, H, N, P), torch.float32, dev)
    lib = load_library()
    scale = 1 if scale_input else 0
    need = int(lib.ssd_forward_dt_varlen_workspace_bytes(ctypes.byref(dims), int(chunk), scale))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr, n, count = None, 0, ctypes.c_int(0)
    if events is not None:
        n = max(len(events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(events) + [None] * (n - len(events))))
    _on_stream(stream, y, final_state, workspace)
    rc = lib.ssd_forward_dt_varlen(ctypes.byref(dims), _ptr(cu_seqlens), int(T), _ptr(x), _ptr(dt), _ptr(dt_bias),
                                   _ptr(A_log), scale, _ptr(B), _ptr(C), _ptr(D), int(chunk), _ptr(init_state),
                                   _ptr(y), _ptr(final_state), _ptr(workspace), ws_bytes,
                                   _stream_handle(stream, dev), arr, n, ctypes.byref(count))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_forward_dt_varlen")
    return y, final_state, (count.value if events is not None else None)


def ssd_forward_dt_workspace_bytes(dims: Dims, chunk: int, scale_input: bool = True) -> int:
    return int(load_library().ssd_forward_dt_workspace_bytes(ctypes.byref(dims), int(chunk),
                                                             1 if scale_input else 0))


def ssd_forward_dt(x, dt, A_log, B, C, D=None, dt_bias=None, scale_input: bool = True,
                   chunk: int = 64, init_state=None, y=None, final_state=None, workspace=None,
                   stream=None):
    """Run ``ssd_forward_dt``: the forward pass with log a = -softplus(dt + dt_bias) exp(A_log)
    formed in the kernels, and (scale_input) the input term scaled by softplus(dt + dt_bias).
    dt [B,T,H] fp32; A_log [H] (scalar decay) or [H,N] (diagonal decay); dt_bias [H] or None.
    Returns (y, final_state)."""
    return _forward_dt(x, dt, A_log, B, C, D, dt_bias, scale_input, chunk, init_state, y,
                       final_state, workspace, stream)[:2]


def ssd_forward_dt_profiled(x, dt, A_log, B, C, D=None, dt_bias=None, scale_input: bool = True,
                            chunk: int = 64, init_state=None, y=None, final_state=None,
                            workspace=None, stream=None, events=()):
    """``ssd_forward_dt_profiled``: as ssd_forward_dt, with per-launch timing events as
    ssd_forward_profiled.  Returns (y, final_state, n_launches)."""
    return _forward_dt(x, dt, A_log, B, C, D, dt_bias, scale_input, chunk, init_state, y,
                       final_state, workspace, stream, events=list(events))


def _forward_dt(x, dt, A_log, B, C, D, dt_bias, scale_input, chunk, init_state, y, final_state,
                workspace, stream, events=None):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [B,T,H,P] and B [B,T,G,N]")
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    decay = SSD_DECAY_DIAG if A_log.dim() == 2 else SSD_DECAY_SCALAR
    dims = Dims(bsz, T, H, G, P, N, _DTYPE_CODE[x.dtype], decay)
    dev = x.device
    _check(x, "x", (bsz, T, H, P), x.dtype, dev)
    _check(dt, "dt", (bsz, T, H), torch.float32, dev)
    _check(A_log, "A_log", (H, N) if decay == SSD_DECAY_DIAG else (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B, "B", (bsz, T, G, N), x.dtype, dev)
    _check(C, "C", (bsz, T, G, N), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (bsz, H, N, P), torch.float32, dev)
    if y is None:
        y = torch.empty((bsz, T, H, P), dtype=x.dtype, device=dev)
    _check(y, "y", (bsz, T, H, P), x.dtype, dev)
    if final_state is True:
        final_state = torch.empty((bsz, H, N, P), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    _check(final_state, "final_state", (bsz, H, N, P), torch.float32, dev)
    lib = load_library()
    scale = 1 if scale_input else 0
    need = int(lib.ssd_forward_dt_workspace_bytes(ctypes.byref(dims), int(chunk), scale))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), scale, _ptr(B),
            _ptr(C), _ptr(D), int(chunk), _ptr(init_state), _ptr(y), _ptr(final_state),
            _ptr(workspace), ws_bytes, _stream_handle(stream, dev))
    _on_stream(stream, y, final_state, workspace)
    if events is None:
        rc = lib.ssd_forward_dt(*args)
        launches = None
    else:
        n = max(len(events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(events) + [None] * (n - len(events))))
        count = ctypes.c_int(0)
        rc = lib.ssd_forward_dt_profiled(*args, arr, n, ctypes.byref(count))
        launches = count.value
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_forward_dt")
    return y, final_state, launches


def ssd_step_dt(state, x_t, dt_t, A_log, B_t, C_t, D=None, dt_bias=None, scale_input: bool = True,
                y_t=None, stream=None):
    """Run ``ssd_step_dt``: one token with the discretisation front-end, ``state`` updated in
    place.  dt_t [B,H] fp32; A_log [H] or [H,N]; other arguments as ssd_step."""
    bsz, H, N, P = state.shape
    G = B_t.shape[1]
    dev = state.device
    decay = SSD_DECAY_DIAG if A_log.dim() == 2 else SSD_DECAY_SCALAR
    if x_t.dtype not in _DTYPE_CODE:
        raise TypeError("x_t must be float32 or bfloat16")
    dims = Dims(bsz, 1, H, G, P, N, _DTYPE_CODE[x_t.dtype], decay)
    _check(state, "state", (bsz, H, N, P), torch.float32, dev)
    _check(x_t, "x_t", (bsz, H, P), x_t.dtype, dev)
    _check(dt_t, "dt_t", (bsz, H), torch.float32, dev)
    _check(A_log, "A_log", (H, N) if decay == SSD_DECAY_DIAG else (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B_t, "B_t", (bsz, G, N), x_t.dtype, dev)
    _check(C_t, "C_t", (bsz, G, N), x_t.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    if y_t is None:
        y_t = torch.empty((bsz, H, P), dtype=x_t.dtype, device=dev)
        _on_stream(stream, y_t)
    _check(y_t, "y_t", (bsz, H, P), x_t.dtype, dev)
    rc = load_library().ssd_step_dt(ctypes.byref(dims), _ptr(state), _ptr(x_t), _ptr(dt_t),
                                    _ptr(dt_bias), _ptr(A_log), 1 if scale_input else 0,
                                    _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(y_t),
                                    _stream_handle(stream, dev))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_step_dt")
    return y_t


def ssd_backward_workspace_bytes(dims: Dims) -> int:
    return int(load_library().ssd_backward_workspace_bytes(ctypes.byref(dims)))


def ssd_backward_profiled(x, log_a, B, C, dy, D=None, init_state=None, dfinal=None, want_dD=True,
                          want_dinit=True, workspace=None, stream=None, events=()):
    """``ssd_backward_profiled``: as ssd_backward, launch k stamping events[2k] and events[2k+1].
    Returns (gradients, n_launches)."""
    return ssd_backward(x, log_a, B, C, dy, D, init_state, dfinal, want_dD, want_dinit, workspace,
                        stream, _events=list(events))


def ssd_backward(x, log_a, B, C, dy, D=None, init_state=None, dfinal=None, want_dD=True,
                 want_dinit=True, workspace=None, stream=None, _events=None):
    """Run ``ssd_backward``: gradients of <dy, y> + <dfinal, final_state> for the forward pass
    on (x, log_a, B, C, D, init_state), scalar or diagonal decay (log_a [B,T,H] or [B,T,H,N]).  Returns a dict: dx (dtype of x), dlog_a,
    dB, dC (fp32), dD (fp32 [H], or None) and dinit (fp32 [B,H,N,P], or None)."""
    dims = dims_for(x, log_a, B)
    dev = x.device
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check(x, "x", (bsz, T, H, P), x.dtype, dev)
    la_shape = (bsz, T, H, N) if dims.decay == SSD_DECAY_DIAG else (bsz, T, H)
    _check(log_a, "log_a", la_shape, torch.float32, dev)
    _check(B, "B", (bsz, T, G, N), x.dtype, dev)
    _check(C, "C", (bsz, T, G, N), x.dtype, dev)
    _check(dy, "dy", (bsz, T, H, P), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (bsz, H, N, P), torch.float32, dev)
    _check(dfinal, "dfinal", (bsz, H, N, P), torch.float32, dev)
    out = dict(dx=torch.empty_like(x), dlog_a=torch.empty(la_shape, dtype=torch.float32, device=dev),
               dB=torch.empty((bsz, T, G, N), dtype=torch.float32, device=dev),
               dC=torch.empty((bsz, T, G, N), dtype=torch.float32, device=dev),
               dD=torch.empty(H, dtype=torch.float32, device=dev) if want_dD else None,
               dinit=torch.empty((bsz, H, N, P), dtype=torch.float32, device=dev) if want_dinit else None)
    lib = load_library()
    need = int(lib.ssd_backward_workspace_bytes(ctypes.byref(dims)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(dims), _ptr(x), _ptr(log_a), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
            _ptr(dy), _ptr(dfinal), _ptr(out["dx"]), _ptr(out["dlog_a"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), _ptr(workspace), ws_bytes,
            _stream_handle(stream, dev))
    _on_stream(stream, workspace, *out.values())
    if _events is None:
        rc = lib.ssd_backward(*args)
    else:
        n = max(len(_events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(_events) + [None] * (n - len(_events))))
        count = ctypes.c_int(0)
        rc = lib.ssd_backward_profiled(*args, arr, n, ctypes.byref(count))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_backward")
    return out if _events is None else (out, count.value)


def ssd_backward_varlen(x, log_a, B, C, dy, cu_seqlens, max_seqlen: int, D=None, init_state=None, dfinal=None,
                        want_dD=True, want_dinit=True, workspace=None, stream=None, events=None):
    """Run ``ssd_backward_varlen``: gradients of <dy, y> + <dfinal, final_states> for
    ssd_forward_varlen on the packed batch (x [T,H,P], log_a [T,H] or [T,H,N], B, C [T,G,N],
    cu_seqlens int64 on the GPU, max_seqlen a bound on every length).  Returns a dict: dx (dtype of
    x), dlog_a, dB, dC (fp32, packed), dD (or None), dinit [nseq,H,N,P] (or None)."""
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or nseq < 0 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor of nseq + 1 offsets on x's device")
    dims = varlen_dims(x, log_a, B, nseq, max_seqlen)
    _check(x, "x", (T, H, P), x.dtype, dev)
    _check(log_a, "log_a", (T, H, N) if dims.decay == SSD_DECAY_DIAG else (T, H), torch.float32, dev)
    _check(B, "B", (T, G, N), x.dtype, dev)
    _check(C, "C", (T, G, N), x.dtype, dev)
    _check(dy, "dy", (T, H, P), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (nseq, H, N, P), torch.float32, dev)
    _check(dfinal, "dfinal", (nseq, H, N, P), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), dlog_a=torch.empty(log_a.shape, **f32), dB=torch.empty((T, G, N), **f32),
               dC=torch.empty((T, G, N), **f32), dD=torch.empty(H, **f32) if want_dD else None,
               dinit=torch.empty((nseq, H, N, P), **f32) if want_dinit else None)
    lib = load_library()
    need = int(lib.ssd_backward_varlen_workspace_bytes(ctypes.byref(dims)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr, n, count = None, 0, ctypes.c_int(0)
    if events is not None:
        n = max(len(events), 2 * SSD_MAX_LAUNCHES)
        arr = (ctypes.c_void_p * n)(*(list(events) + [None] * (n - len(events))))
    _on_stream(stream, workspace, *out.values())
    rc = lib.ssd_backward_varlen(ctypes.byref(dims), _ptr(cu_seqlens), int(T), _ptr(x), _ptr(log_a), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(init_state), _ptr(dy), _ptr(dfinal), _ptr(out["dx"]),
                                 _ptr(out["dlog_a"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                                 _ptr(out["dinit"]), _ptr(workspace), ws_bytes, _stream_handle(stream, dev), arr, n,
                                 ctypes.byref(count))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_backward_varlen")
    return out


def ssd_backward_dt(x, dt, A_log, B, C, dy, D=None, dt_bias=None, scale_input: bool = True,
                    init_state=None, dfinal=None, want_dD=True, want_dinit=True, workspace=None,
                    stream=None):
    """Run ``ssd_backward_dt``: gradients of <dy, y> + <dfinal, final_state> for ssd_forward_dt
    (scalar decay with A_log [H], diagonal with A_log [H,N]).  Returns a dict: dx (dtype of x),
    ddt [B,T,H], dA_log (A_log's shape), ddt_bias [H] (or None without dt_bias), dB, dC (fp32),
    dD (or None), dinit (or None)."""
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16")
    decay = SSD_DECAY_DIAG if A_log.dim() == 2 else SSD_DECAY_SCALAR
    dims = Dims(bsz, T, H, G, P, N, _DTYPE_CODE[x.dtype], decay)
    dev = x.device
    _check(x, "x", (bsz, T, H, P), x.dtype, dev)
    _check(dt, "dt", (bsz, T, H), torch.float32, dev)
    _check(A_log, "A_log", (H, N) if decay == SSD_DECAY_DIAG else (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B, "B", (bsz, T, G, N), x.dtype, dev)
    _check(C, "C", (bsz, T, G, N), x.dtype, dev)
    _check(dy, "dy", (bsz, T, H, P), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (bsz, H, N, P), torch.float32, dev)
    _check(dfinal, "dfinal", (bsz, H, N, P), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty((bsz, T, H), **f32), dA_log=torch.empty(A_log.shape, **f32),
               ddt_bias=torch.empty(H, **f32) if dt_bias is not None else None,
               dB=torch.empty((bsz, T, G, N), **f32), dC=torch.empty((bsz, T, G, N), **f32),
               dD=torch.empty(H, **f32) if want_dD else None,
               dinit=torch.empty((bsz, H, N, P), **f32) if want_dinit else None)
    lib = load_library()
    scale = 1 if scale_input else 0
    need = int(lib.ssd_backward_dt_workspace_bytes(ctypes.byref(dims), scale))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _on_stream(stream, workspace, *out.values())
    rc = lib.ssd_backward_dt(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), scale,
                             _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(dy), _ptr(dfinal),
                             _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA_log"]),
                             _ptr(out["ddt_bias"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                             _ptr(out["dinit"]), _ptr(workspace), ws_bytes, _stream_handle(stream, dev))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_backward_dt")
    return out


def ssd_backward_dt_varlen(x, dt, A_log, B, C, dy, cu_seqlens, max_seqlen: int, D=None, dt_bias=None,
                           scale_input: bool = True, init_state=None, dfinal=None, want_dD=True, want_dinit=True,
                           workspace=None, stream=None):
    """Run ``ssd_backward_dt_varlen``: the gradients of ssd_forward_dt_varlen on a packed batch
    (x [T,H,P], dt [T,H], B, C [T,G,N], cu_seqlens int64 on the GPU).  Returns a dict as
    ssd_backward_dt's, with dx, ddt, dB, dC packed and dinit [nseq,H,N,P]."""
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or nseq < 0 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor of nseq + 1 offsets on x's device")
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16")
    decay = SSD_DECAY_DIAG if A_log.dim() == 2 else SSD_DECAY_SCALAR
    dims = Dims(int(nseq), int(max_seqlen), H, G, P, N, _DTYPE_CODE[x.dtype], decay)
    _check(x, "x", (T, H, P), x.dtype, dev)
    _check(dt, "dt", (T, H), torch.float32, dev)
    _check(A_log, "A_log", (H, N) if decay == SSD_DECAY_DIAG else (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B, "B", (T, G, N), x.dtype, dev)
    _check(C, "C", (T, G, N), x.dtype, dev)
    _check(dy, "dy", (T, H, P), x.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(init_state, "init_state", (nseq, H, N, P), torch.float32, dev)
    _check(dfinal, "dfinal", (nseq, H, N, P), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty((T, H), **f32), dA_log=torch.empty(A_log.shape, **f32),
               ddt_bias=torch.empty(H, **f32) if dt_bias is not None else None,
               dB=torch.empty((T, G, N), **f32), dC=torch.empty((T, G, N), **f32),
               dD=torch.empty(H, **f32) if want_dD else None,
               dinit=torch.empty((nseq, H, N, P), **f32) if want_dinit else None)
    lib = load_library()
    scale = 1 if scale_input else 0
    need = int(lib.ssd_backward_dt_varlen_workspace_bytes(ctypes.byref(dims), scale))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _on_stream(stream, workspace, *out.values())
    rc = lib.ssd_backward_dt_varlen(ctypes.byref(dims), _ptr(cu_seqlens), int(T), _ptr(x), _ptr(dt), _ptr(dt_bias),
                                    _ptr(A_log), scale, _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(dy),
                                    _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA_log"]),
                                    _ptr(out["ddt_bias"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                                    _ptr(out["dinit"]), _ptr(workspace), ws_bytes, _stream_handle(stream, dev))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_backward_dt_varlen")
    return out


def ssd_step(state, x_t, log_a_t, B_t, C_t, D=None, y_t=None, stream=None):
    """Run ``ssd_step``: one token for every (batch, head), ``state`` updated in place.
    state [B,H,N,P] fp32; x_t [B,H,P]; log_a_t [B,H] or [B,H,N]; B_t, C_t [B,G,N]."""
    bsz, H, N, P = state.shape
    G = B_t.shape[1]
    dev = state.device
    decay = SSD_DECAY_DIAG if log_a_t.dim() == 3 else SSD_DECAY_SCALAR
    if x_t.dtype not in _DTYPE_CODE:
        raise TypeError("x_t must be float32 or bfloat16")
    dims = Dims(bsz, 1, H, G, P, N, _DTYPE_CODE[x_t.dtype], decay)
    _check(state, "state", (bsz, H, N, P), torch.float32, dev)
    _check(x_t, "x_t", (bsz, H, P), x_t.dtype, dev)
    _check(log_a_t, "log_a_t", (bsz, H, N) if decay == SSD_DECAY_DIAG else (bsz, H),
           torch.float32, dev)
    _check(B_t, "B_t", (bsz, G, N), x_t.dtype, dev)
    _check(C_t, "C_t", (bsz, G, N), x_t.dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    if y_t is None:
        y_t = torch.empty((bsz, H, P), dtype=x_t.dtype, device=dev)
        _on_stream(stream, y_t)
    _check(y_t, "y_t", (bsz, H, P), x_t.dtype, dev)
    rc = load_library().ssd_step(ctypes.byref(dims), _ptr(state), _ptr(x_t), _ptr(log_a_t),
                                 _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(y_t),
                                 _stream_handle(stream, dev))
    if rc != SSD_OK:
        raise SSDError(rc, "ssd_step")
    return y_t
