"""ctypes loader for the fp64 adjoint in ``ssd_oracle_bwd.c`` (test infrastructure only).

The gradient of L(x, log a, B, C, D, init) = <dy, y> + <dfinal, final> through the recurrence
of ``ssd_oracle.c``, swept backwards by the chain rule (see the C file's header).  Inputs are
float64 numpy arrays widened exactly from the stored inputs.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .recurrence import BUILD_DIR, build as _build, default_threads

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle_bwd.c")
LIBRARY = os.path.join(BUILD_DIR, "libssd_oracle_bwd.so")

_f64p = ctypes.POINTER(ctypes.c_double)


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the adjoint with gcc (-O2, OpenMP, no fast-math) into a shared library."""
    return _build(source, output)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_f64p)


def _as_f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


class Adjoint:
    """Handle on one compiled copy of the adjoint."""

    def __init__(self, library: str | None = None):
        if library is None:
            library = LIBRARY
            if not os.path.exists(library) or os.path.getmtime(library) < os.path.getmtime(SOURCE):
                build()
        self.library = library
        lib = ctypes.CDLL(library)
        fn = lib.ssd_oracle_backward
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int] + [_f64p] * 14 + [ctypes.c_int]
        self._fn = fn

    def backward(self, x, log_a, Bm, Cm, D, init_state, dy, dfinal=None, nthreads: int | None = None):
        """Gradients of <dy, y> + <dfinal, final> with respect to every input.

        x [B,T,H,P]; log_a [B,T,H] or [B,T,H,N]; Bm, Cm [B,T,G,N]; D [H] or None; init_state
        [B,H,N,P] or None; dy [B,T,H,P]; dfinal [B,H,N,P] or None.  Returns a dict of float64
        arrays: dx, dlog_a, dB, dC, dD (zeros [H] when D is None) and dinit.
        """
        x, log_a, Bm, Cm, dy = (_as_f64(a) for a in (x, log_a, Bm, Cm, dy))
        D, init_state, dfinal = _as_f64(D), _as_f64(init_state), _as_f64(dfinal)
        nb, T, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        if log_a.shape == (nb, T, H):
            diag = 0
        elif log_a.shape == (nb, T, H, N):
            diag = 1
        else:
            raise ValueError("log_a must be [B,T,H] or [B,T,H,N]")
        if dy.shape != x.shape or Cm.shape != Bm.shape or Bm.shape[:2] != (nb, T) or H % G:
            raise ValueError("shapes do not match")
        out = dict(dx=np.empty_like(x), dlog_a=np.empty_like(log_a), dB=np.empty_like(Bm),
                   dC=np.empty_like(Cm), dD=np.zeros(H), dinit=np.empty((nb, H, N, P)))
        rc = self._fn(nb, T, H, G, P, N, diag, _ptr(x), _ptr(log_a), _ptr(Bm), _ptr(Cm), _ptr(D),
                      _ptr(init_state), _ptr(dy), _ptr(dfinal), _ptr(out["dx"]), _ptr(out["dlog_a"]),
                      _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]),
                      nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("ssd_oracle_backward failed with code %d" % rc)
        return out


_DEFAULT: Adjoint | None = None


def default_adjoint() -> Adjoint:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Adjoint()
    return _DEFAULT


def backward(*args, **kwargs):
    """``Adjoint.backward`` on the default compiled adjoint."""
    return default_adjoint().backward(*args, **kwargs)
