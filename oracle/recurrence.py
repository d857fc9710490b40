"""ctypes loader for the fp64 C recurrence in ``ssd_oracle.c`` (test infrastructure only).

The recurrence is the exact operator the chunked SSD forward computes (llms.blog "State
Space Models and Mamba": "Continuous-to-Discrete Discretization" for h_t = A h_{t-1} + B x_t,
y_t = C h_t + D x_t, with A_t = a_t I from "The SSD Theoretical Equivalence").  Inputs are
float64 numpy arrays: the caller widens the stored inputs (fp32 values or bf16 bit patterns)
exactly, so a comparison with the GPU path measures the kernels' arithmetic only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle.c")
BUILD_DIR = os.path.join(_HERE, "_build")
LIBRARY = os.path.join(BUILD_DIR, "libssd_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math) into a shared library."""
    os.makedirs(os.path.dirname(output), exist_ok=True)
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def default_threads() -> int:
    """Threads the oracle uses: OMP_NUM_THREADS if set, else the CPUs this process may use."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.strip().isdigit() and int(env) > 0:
        return int(env)
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_f64p)


def _as_f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """Handle on one compiled copy of the C oracle."""

    def __init__(self, library: str | None = None):
        if library is None:
            library = LIBRARY
            if (not os.path.exists(library)
                    or os.path.getmtime(library) < os.path.getmtime(SOURCE)):
                build()
        self.library = library
        lib = ctypes.CDLL(library)
        fn = lib.ssd_oracle_forward
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int] + [_f64p] * 8 + [ctypes.c_int]
        self._fn = fn
        self._lib = lib

    def forward(self, x, log_a, Bm, Cm, D=None, init_state=None, want_final=True,
                nthreads: int | None = None):
        """Run the recurrence.

        x [B,T,H,P]; log_a [B,T,H] (scalar decay) or [B,T,H,N] (per-state-dim decay);
        Bm, Cm [B,T,G,N]; D [H] or None; init_state [B,H,N,P] or None.
        Returns (y [B,T,H,P], final_state [B,H,N,P] or None), both float64.
        """
        x, log_a, Bm, Cm = (_as_f64(a) for a in (x, log_a, Bm, Cm))
        D, init_state = _as_f64(D), _as_f64(init_state)
        if x.ndim != 4 or Bm.ndim != 4 or Cm.shape != Bm.shape:
            raise ValueError("x must be [B,T,H,P] and Bm, Cm [B,T,G,N] with equal shapes")
        nb, T, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        if Bm.shape[:2] != (nb, T) or H % G != 0:
            raise ValueError("Bm/Cm leading dims must match x and G must divide H")
        if log_a.shape == (nb, T, H):
            diag = 0
        elif log_a.shape == (nb, T, H, N):
            diag = 1
        else:
            raise ValueError("log_a must be [B,T,H] or [B,T,H,N], got %s" % (log_a.shape,))
        if D is not None and D.shape != (H,):
            raise ValueError("D must be [H]")
        if init_state is not None and init_state.shape != (nb, H, N, P):
            raise ValueError("init_state must be [B,H,N,P]")
        y = np.empty((nb, T, H, P), dtype=np.float64)
        final = np.empty((nb, H, N, P), dtype=np.float64) if want_final else None
        rc = self._fn(nb, T, H, G, P, N, diag, _ptr(x), _ptr(log_a), _ptr(Bm), _ptr(Cm),
                      _ptr(D), _ptr(init_state), _ptr(y), _ptr(final),
                      nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("ssd_oracle_forward failed with code %d" % rc)
        return y, final


_DEFAULT: Oracle | None = None


def default_oracle() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def forward(*args, **kwargs):
    """``Oracle.forward`` on the default compiled oracle."""
    return default_oracle().forward(*args, **kwargs)
