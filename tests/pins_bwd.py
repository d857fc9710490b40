"""Pins for the CPU oracle's backward pass (oracle/backward.py): checks against facts that do not
come from the adjoint's own code.

Every pin takes the forward oracle handle ``orc`` and an adjoint handle ``adj`` (anything with
``backward(x, log_a, Bm, Cm, D, init_state, dy, dfinal)`` returning the gradient dict), and
raises AssertionError when they disagree with:
  * central finite differences of L = <dy, y> + <dfinal, final>, evaluated with the forward
    oracle alone, along a random direction in each input;
  * exact linearity: y and final are linear in x, B, C, D and init separately, so
    L(theta + v) - L(theta) equals <dL/dtheta, v> up to rounding, with no step size;
  * closed forms at a = 1 (log a = 0): the state is the running sum, so
    dL/dh_t = dfinal + sum_{s >= t} C_s dy_s^T, a reverse cumulative sum.
"""
from __future__ import annotations

import numpy as np

from pins import _close


def _problem(rng, nb=2, T=9, H=4, G=2, P=3, N=5, diag=False):
    x = rng.standard_normal((nb, T, H, P))
    Bm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    shape = (nb, T, H, N) if diag else (nb, T, H)
    log_a = -np.log1p(np.exp(rng.standard_normal(shape)))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((nb, H, N, P))
    dy = rng.standard_normal((nb, T, H, P))
    dfin = rng.standard_normal((nb, H, N, P))
    return dict(x=x, log_a=log_a, Bm=Bm, Cm=Cm, D=D, init=h0), dy, dfin


def _loss(orc, inp, dy, dfin):
    y, fin = orc.forward(inp["x"], inp["log_a"], inp["Bm"], inp["Cm"], inp["D"], inp["init"])
    return float(np.sum(dy * y) + np.sum(dfin * fin))


def _grads(adj, inp, dy, dfin):
    return adj.backward(inp["x"], inp["log_a"], inp["Bm"], inp["Cm"], inp["D"], inp["init"], dy, dfin)


GRAD_OF = dict(x="dx", log_a="dlog_a", Bm="dB", Cm="dC", D="dD", init="dinit")


def pin_bwd_finite_differences(orc, adj):
    """Every gradient along a random direction against a central difference (step 1e-6, fp64;
    error O(step^2) and O(1e-16 / step), so agreement to ~1e-8 relative)."""
    for diag in (False, True):
        rng = np.random.default_rng(61 + diag)
        inp, dy, dfin = _problem(rng, diag=diag)
        g = _grads(adj, inp, dy, dfin)
        eps = 1e-6
        for name, gname in GRAD_OF.items():
            v = rng.standard_normal(inp[name].shape)
            plus = dict(inp, **{name: inp[name] + eps * v})
            minus = dict(inp, **{name: inp[name] - eps * v})
            fd = (_loss(orc, plus, dy, dfin) - _loss(orc, minus, dy, dfin)) / (2 * eps)
            an = float(np.sum(g[gname] * v))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), "%s (diag=%d): fd %.12g adjoint %.12g" % (
                gname, diag, fd, an)


def pin_bwd_linear_inputs_exact(orc, adj):
    """y and final are linear in each of x, B, C, D and init (the others fixed), so a finite
    step of any size gives the directional derivative exactly: L(theta + v) - L(theta) =
    <grad, v> to rounding."""
    rng = np.random.default_rng(63)
    inp, dy, dfin = _problem(rng, T=12)
    g = _grads(adj, inp, dy, dfin)
    base = _loss(orc, inp, dy, dfin)
    for name in ("x", "Bm", "Cm", "D", "init"):
        v = rng.standard_normal(inp[name].shape)
        step = _loss(orc, dict(inp, **{name: inp[name] + v}), dy, dfin) - base
        an = float(np.sum(g[GRAD_OF[name]] * v))
        assert abs(step - an) <= 1e-11 * max(1.0, abs(step)), "%s: step %.15g adjoint %.15g" % (name, step, an)


def pin_bwd_a_one_closed_form(orc, adj):
    """a = 1 (log a = 0): dL/dh_t = dfinal + sum_{s >= t} C_s dy_s^T (a reverse cumulative sum),
    so dx_t = (dL/dh_t)^T B_t + D dy_t, dB_t = (dL/dh_t) x_t, dinit = dL/dh_0, and
    dlog a_t = <dL/dh_t, h_{t-1}> with h_{t-1} = h_0 + sum_{s < t} B_s x_s^T."""
    rng = np.random.default_rng(64)
    inp, dy, dfin = _problem(rng, nb=1, T=10, H=2, G=1, P=3, N=4)
    inp["log_a"] = np.zeros_like(inp["log_a"])
    g = _grads(adj, inp, dy, dfin)
    x, Bm, Cm, D, h0 = inp["x"], inp["Bm"], inp["Cm"], inp["D"], inp["init"]
    for h in range(x.shape[2]):
        outer_cd = Cm[0, :, 0, :, None] * dy[0, :, h, None, :]               # [T, N, P]
        Gt = dfin[0, h][None] + np.cumsum(outer_cd[::-1], axis=0)[::-1]      # dL/dh_t
        outer_bx = Bm[0, :, 0, :, None] * x[0, :, h, None, :]
        hprev = h0[0, h][None] + np.concatenate([np.zeros((1,) + outer_bx.shape[1:]),
                                                 np.cumsum(outer_bx, axis=0)[:-1]])
        _close(g["dx"][0, :, h], np.einsum("tnp,tn->tp", Gt, Bm[0, :, 0]) + D[h] * dy[0, :, h], "a=1 dx")
        _close(g["dinit"][0, h], Gt[0], "a=1 dinit")
        _close(g["dlog_a"][0, :, h], np.einsum("tnp,tnp->t", Gt, hprev), "a=1 dlog_a")
    # B and C are shared by both heads: their gradients sum over the heads
    want_dB = sum(np.einsum("tnp,tp->tn", dfin[0, h][None] + np.cumsum(
        (Cm[0, :, 0, :, None] * dy[0, :, h, None, :])[::-1], axis=0)[::-1], x[0, :, h]) for h in range(2))
    _close(g["dB"][0, :, 0], want_dB, "a=1 dB (summed over the group's heads)")
    _close(g["dD"], np.einsum("bthp,bthp->h", dy, x), "dD")


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_linear_inputs_exact, pin_bwd_a_one_closed_form]


def pin_bwd_dt_finite_differences(orc, adj, disc):
    """The discretised form's gradients (disc.backward_dt on the adjoint adj) against central
    differences of L = <dy, y> + <dfinal, final> evaluated with disc.forward_dt on the forward
    oracle alone, along a random direction in each of x, dt, A_log, dt_bias, B, C, D and init;
    with and without the input scale, for one rate per head (A_log [H]) and one per head and state
    dimension (A_log [H,N])."""
    rng = np.random.default_rng(81)
    nb, T, H, G, P, N = 2, 9, 4, 2, 3, 5
    x = rng.standard_normal((nb, T, H, P))
    Bm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    base = dict(x=x, dt=rng.standard_normal((nb, T, H)) - 1.0, dt_bias=rng.standard_normal(H) * 0.5, Bm=Bm, Cm=Cm,
                D=rng.standard_normal(H), init=rng.standard_normal((nb, H, N, P)))
    dy = rng.standard_normal((nb, T, H, P))
    dfin = rng.standard_normal((nb, H, N, P))
    names = dict(x="dx", dt="ddt", A_log="dA_log", dt_bias="ddt_bias", Bm="dB", Cm="dC", D="dD", init="dinit")
    for diag in (False, True):
        inp = dict(base, A_log=rng.uniform(0.0, 2.0, (H, N) if diag else H))
        for scale in (True, False):
            def loss(d):
                y, fin = disc.forward_dt(orc, d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"],
                                         dt_bias=d["dt_bias"], scale_input=scale, init_state=d["init"], diag=diag)
                return float(np.sum(dy * y) + np.sum(dfin * fin))
            g = disc.backward_dt(adj, inp["x"], inp["dt"], inp["A_log"], inp["Bm"], inp["Cm"], inp["D"],
                                 dt_bias=inp["dt_bias"], scale_input=scale, init_state=inp["init"], dy=dy,
                                 dfinal=dfin, diag=diag)
            eps = 1e-6
            for name, gname in names.items():
                v = rng.standard_normal(np.shape(inp[name]))
                fd = (loss(dict(inp, **{name: inp[name] + eps * v})) - loss(dict(inp, **{name: inp[name] - eps * v}))) \
                    / (2 * eps)
                an = float(np.sum(g[gname] * v))
                assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), "%s (diag=%d, scale=%d): fd %.12g chain rule %.12g" % (
                    gname, diag, scale, fd, an)


BWD_DT_PINS = [pin_bwd_dt_finite_differences]
