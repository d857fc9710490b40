"""Packed variable-length batches in the oracle (test infrastructure only: the tests, the smoke
check and the CPU-baseline leg of the benchmark may call it; the product path never does).

A packed batch holds nseq sequences one after another on the token axis: sequence i is tokens
cu_seqlens[i] .. cu_seqlens[i+1] - 1 of x [T,H,P], log_a [T,H] or [T,H,N], B, C [T,G,N] and y.
Each sequence runs the recurrence by itself, from its own initial state (init_states[i], zeros when
absent) to its own final state; nothing passes from one sequence to the next.  That is a batch of
independent sequences (llms.blog "State Space Models and Mamba": the recurrence of "Continuous-to-
Discrete Discretization" starts from its initial hidden state for every input sequence), stored
packed instead of padded.  Each sequence goes through the fp64 recurrence of ``ssd_oracle.c``.
"""
from __future__ import annotations

import numpy as np


def check_cu_seqlens(cu_seqlens, total):
    """cu_seqlens as int64, checked: starts at 0, never decreases, ends at total."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != total:
        raise ValueError("cu_seqlens must start at 0, never decrease and end at the token count")
    return cu


def forward_varlen(orc, x, log_a, Bm, Cm, cu_seqlens, D=None, init_states=None, want_final=True):
    """y [T,H,P] and the final states [nseq,H,N,P] (float64) of a packed batch.  ``orc`` is an oracle
    handle (``oracle.Oracle``); init_states [nseq,H,N,P] or None."""
    x = np.asarray(x, dtype=np.float64)
    log_a = np.asarray(log_a, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    T, H, P = x.shape
    N = Bm.shape[2]
    cu = check_cu_seqlens(cu_seqlens, T)
    nseq = cu.size - 1
    y = np.zeros((T, H, P))
    finals = np.zeros((nseq, H, N, P)) if want_final else None
    for i in range(nseq):
        s, e = int(cu[i]), int(cu[i + 1])
        init = None if init_states is None else np.asarray(init_states, dtype=np.float64)[i:i + 1]
        if e == s:
            if want_final and init is not None:
                finals[i] = init[0]
            continue
        yi, fi = orc.forward(x[None, s:e], log_a[None, s:e], Bm[None, s:e], Cm[None, s:e], D, init, want_final)
        y[s:e] = yi[0]
        if want_final:
            finals[i] = fi[0]
    return y, finals


def backward_varlen(adj, x, log_a, Bm, Cm, cu_seqlens, D=None, init_states=None, dy=None, dfinal=None):
    """Gradients of <dy, y> + <dfinal, finals> for ``forward_varlen``: every sequence through the
    fp64 adjoint of ``ssd_oracle_bwd.c`` (``adj``, an ``oracle.backward.Adjoint``) by itself.
    Each token's dx, dlog_a, dB and dC come from its own sequence; dD sums over all of them; dinit
    [nseq,H,N,P] is each sequence's (dfinal[i] for an empty one).  Returns a dict of float64
    arrays."""
    x = np.asarray(x, dtype=np.float64)
    log_a = np.asarray(log_a, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, H, P = x.shape
    N = Bm.shape[2]
    cu = check_cu_seqlens(cu_seqlens, T)
    nseq = cu.size - 1
    out = dict(dx=np.zeros_like(x), dlog_a=np.zeros_like(log_a), dB=np.zeros_like(Bm), dC=np.zeros_like(Cm),
               dD=np.zeros(H), dinit=np.zeros((nseq, H, N, P)))
    for i in range(nseq):
        s = int(cu[i])
        e = int(cu[i + 1])
        fin = None if dfinal is None else np.asarray(dfinal, dtype=np.float64)[i:i + 1]
        if e == s:
            if fin is not None:
                out["dinit"][i] = fin[0]
            continue
        init = None if init_states is None else np.asarray(init_states, dtype=np.float64)[i][None]
        g = adj.backward(x[None, s:e], log_a[None, s:e], Bm[None, s:e], Cm[None, s:e], D, init, dy[None, s:e], fin)
        for k in ("dx", "dlog_a", "dB", "dC"):
            out[k][s:e] = g[k][0]
        out["dD"] += g["dD"]
        out["dinit"][i] = g["dinit"][0]
    return out
