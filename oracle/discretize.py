"""Discretisation front-end of the oracle (test infrastructure only: the tests, the smoke check
and the CPU-baseline leg of the benchmark may call it; the product path never does).

What it computes, in float64, from the step-size pre-activation dt:

    Delta_t  = softplus(dt[b,t,h] + dt_bias[h])          (dt_bias optional, 0 when absent)
    A        = -exp(A_log)                               [H] scalar decay, or [H,N] per state dim
    log a_t  = Delta_t * A                               [B,T,H] or [B,T,H,N]
    input term of the recurrence: Delta_t B_t x_t^T      (scale_input; else B_t x_t^T)
    skip term: D x_t with the raw x_t

Sources (State Space Models and Mamba, llms.blog): the zero-order-hold rule A-bar = exp(Delta A)
of "Continuous-to-Discrete Discretization"; the input-dependent step size (softplus of a
learned bias plus a projection of the token), A-bar_t = exp(Delta_t A) and B-bar_t = Delta_t B_t
of "The Selection Mechanism".  A = -exp(A_log) is the parameterisation the synthetic workloads
state (log a_t = -softplus(dt_t) exp(A_log)); it keeps A negative, so a_t lies in (0, 1].

The recurrence with B-bar_t = Delta_t B_t equals the plain recurrence run on the scaled input
Delta_t x_t (Delta_t is one number per (token, head)), with the skip term added on the raw x
afterwards; that is how ``forward_dt`` evaluates it, on the fp64 recurrence of ``ssd_oracle.c``.
"""
from __future__ import annotations

import numpy as np


def softplus(v):
    """log(1 + e^v) in float64 without overflow (numpy's logaddexp(0, v))."""
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


def discretize(dt, A_log, dt_bias=None, diag=False):
    """(Delta [B,T,H], log a [B,T,H] or [B,T,H,N]) from dt [B,T,H], A_log [H] or [H,N] and an
    optional dt_bias [H]."""
    dt = np.asarray(dt, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    if dt.ndim != 3:
        raise ValueError("dt must be [B,T,H]")
    H = dt.shape[2]
    v = dt if dt_bias is None else dt + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    delta = softplus(v)
    A = -np.exp(A_log)
    if diag:
        if A_log.ndim != 2 or A_log.shape[0] != H:
            raise ValueError("A_log must be [H,N] for per-state-dim decay")
        log_a = delta[..., None] * A[None, None, :, :]
    else:
        if A_log.shape != (H,):
            raise ValueError("A_log must be [H] for scalar decay")
        log_a = delta * A[None, None, :]
    return delta, log_a


def forward_dt(orc, x, dt, A_log, Bm, Cm, D=None, dt_bias=None, scale_input=True, init_state=None,
               want_final=True, diag=False, nthreads=None):
    """The recurrence in its discretised form: y [B,T,H,P] and the final state [B,H,N,P]
    (float64).  ``orc`` is an oracle handle (``oracle.Oracle``)."""
    x = np.asarray(x, dtype=np.float64)
    delta, log_a = discretize(dt, A_log, dt_bias, diag)
    xin = x * delta[..., None] if scale_input else x
    y, final = orc.forward(xin, log_a, Bm, Cm, None, init_state, want_final, nthreads=nthreads)
    if D is not None:
        y = y + np.asarray(D, dtype=np.float64)[None, None, :, None] * x
    return y, final


def sigmoid(v):
    """1 / (1 + e^-v), the derivative of softplus, in float64."""
    return 0.5 * (1.0 + np.tanh(0.5 * np.asarray(v, dtype=np.float64)))


def backward_dt(adj, x, dt, A_log, Bm, Cm, D=None, dt_bias=None, scale_input=True, init_state=None, dy=None,
                dfinal=None, diag=False):
    """Gradients of <dy, y> + <dfinal, final> for ``forward_dt``, by the chain rule through the
    discretisation on top of the recurrence's adjoint ``adj`` (``oracle.backward``): with
    u = dt + bias, Delta = softplus(u), log a = Delta A (A = -exp(A_log), [H] or with ``diag``
    [H,N]) and the recurrence run on x_in = Delta x (scale_input) or x,
        dx       = Delta dx_in (or dx_in) + D dy
        dDelta   = sum_n dlog_a A + sum_p dx_in x   (the sum over n for diag only; the second term
                                                      with scale_input only)
        ddt      = dDelta sigmoid(u),   ddt_bias = sum_{b,t} ddt,   dA_log = sum_{b,t} dlog_a log a
        dD       = sum_{b,t,p} dy x
    and dB, dC, dinit as the adjoint gives them.  Returns a dict of float64 arrays."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    delta, log_a = discretize(dt, A_log, dt_bias, diag)
    u = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        u = u + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    xin = (x * delta[..., None]) if scale_input else x
    g = adj.backward(xin, log_a, Bm, Cm, None, init_state, dy, dfinal)
    dxin = g["dx"]
    dx = dxin * delta[..., None] if scale_input else dxin.copy()
    if D is not None:
        dx = dx + np.asarray(D, dtype=np.float64)[None, None, :, None] * dy
    if diag:
        ddelta = np.einsum("bthn,hn->bth", g["dlog_a"], A)
    else:
        ddelta = g["dlog_a"] * A[None, None, :]
    if scale_input:
        ddelta = ddelta + np.sum(dxin * x, axis=-1)
    ddt = ddelta * sigmoid(u)
    return dict(dx=dx, ddt=ddt, ddt_bias=ddt.sum(axis=(0, 1)), dA_log=np.sum(g["dlog_a"] * log_a, axis=(0, 1)),
                dB=g["dB"], dC=g["dC"], dD=np.einsum("bthp,bthp->h", dy, x), dinit=g["dinit"])
