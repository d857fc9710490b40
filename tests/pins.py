"""Pins for the CPU oracle: checks against facts the pages and the mathematics fix, each
independent of the oracle's own code.

Every pin takes an oracle handle (anything with ``forward(x, log_a, Bm, Cm, D, init_state)``
returning ``(y, final_state)`` in float64) and raises AssertionError when the oracle
disagrees.  ``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on copies of the oracle with a planted mistake and requires that some pin fails.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RTOL = 1e-10


def _close(got, want, what, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, "%s: shape %s != %s" % (what, got.shape, want.shape)
    scale = max(1.0, float(np.abs(want).max()) if want.size else 1.0)
    err = float(np.abs(got - want).max()) if want.size else 0.0
    assert err <= rtol * scale, "%s: max abs error %.3e (scale %.3e)" % (what, err, scale)


def _problem(rng, nb=2, T=40, H=4, G=2, P=5, N=3, diag=False, decay_scale=1.0):
    x = rng.standard_normal((nb, T, H, P))
    Bm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    shape = (nb, T, H, N) if diag else (nb, T, H)
    log_a = -decay_scale * np.log1p(np.exp(rng.standard_normal(shape)))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((nb, H, N, P))
    return x, log_a, Bm, Cm, D, h0


# --- hand-worked examples -------------------------------------------------------------
def _handworked(orc, name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    a = np.array(g["a"], dtype=np.float64)
    x = np.array(g["x"], dtype=np.float64)[None, :, None, :]
    Bm = np.array(g["B"], dtype=np.float64)[None, :, None, :]
    Cm = np.array(g["C"], dtype=np.float64)[None, :, None, :]
    log_a = np.log(a)[None, :, None] if a.ndim == 1 else np.log(a)[None, :, None, :]
    D = np.array([g["D"]], dtype=np.float64)
    h0 = np.array(g["init_state"], dtype=np.float64)[None, None]
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    _close(y[0, :, 0, :], g["y"], name + " y", rtol=1e-14)
    _close(fin[0, 0], g["final_state"], name + " final", rtol=1e-14)


def pin_handworked_scalar(orc):
    """Three recurrence steps worked by hand (tests/golden/handworked_scalar.json)."""
    _handworked(orc, "handworked_scalar.json")


def pin_handworked_diag(orc):
    """Three diagonal-decay steps worked by hand (tests/golden/handworked_diag.json)."""
    _handworked(orc, "handworked_diag.json")


# --- the matrix (attention) form -------------------------------------------------------
def _materialized(x, log_a, Bm, Cm, D, h0):
    """Y = M X + D x + (init term), with M built entry by entry from direct products of the
    decays:  M_ij = C_i^T (prod_{k=j+1..i} A_k) B_j for i >= j, 0 otherwise (llms.blog,
    "The SSD Theoretical Equivalence"; diagonal A_k per "On Structured State-Space Duality").
    The initial state enters as C_i^T (prod_{k=0..i} A_k) h_0.  No prefix sums are used."""
    nb, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    diag = log_a.ndim == 4
    a = np.exp(log_a)
    y = np.zeros_like(x)
    fin = np.zeros((nb, H, N, P))
    for b in range(nb):
        for h in range(H):
            g = h // (H // G)
            # decay products as length-N vectors (scalar decay repeated over n)
            def prod(j0, j1):  # product of A_k for k in [j0, j1]
                v = np.ones(N)
                for k in range(j0, j1 + 1):
                    v = v * (a[b, k, h] if diag else np.full(N, a[b, k, h]))
                return v
            M = np.zeros((T, T))
            for i in range(T):
                for j in range(i + 1):
                    M[i, j] = np.sum(Cm[b, i, g] * prod(j + 1, i) * Bm[b, j, g])
            X = x[b, :, h, :]
            Y = M @ X + D[h] * X
            for i in range(T):
                Y[i] += (Cm[b, i, g] * prod(0, i)) @ h0[b, h]
            y[b, :, h, :] = Y
            S = prod(0, T - 1)[:, None] * h0[b, h]
            for j in range(T):
                S = S + (prod(j + 1, T - 1) * Bm[b, j, g])[:, None] * X[j][None, :]
            fin[b, h] = S
    return y, fin


def pin_materialized_scalar(orc):
    """Recurrence == semiseparable matrix form, scalar decay, with skip and init state."""
    rng = np.random.default_rng(11)
    prob = _problem(rng, nb=2, T=33, H=4, G=2, P=5, N=3)
    y, fin = orc.forward(*prob)
    ym, fm = _materialized(*prob)
    _close(y, ym, "materialized scalar y")
    _close(fin, fm, "materialized scalar final")


def pin_materialized_diag(orc):
    """Recurrence == matrix form with one decay per state dimension."""
    rng = np.random.default_rng(12)
    prob = _problem(rng, nb=1, T=29, H=4, G=2, P=4, N=3, diag=True)
    y, fin = orc.forward(*prob)
    ym, fm = _materialized(*prob)
    _close(y, ym, "materialized diag y")
    _close(fin, fm, "materialized diag final")


# --- closed forms ----------------------------------------------------------------------
def pin_a_one(orc):
    """a = 1 (log a = 0): cumulative linear attention,
    y_t = C_t^T (h_0 + sum_{j<=t} B_j x_j^T) + D x_t and final = h_0 + B^T X
    (the Delta -> 0 limit A -> I of llms.blog "The Selection Mechanism")."""
    rng = np.random.default_rng(13)
    x, _, Bm, Cm, D, h0 = _problem(rng, nb=2, T=37, H=4, G=2, P=6, N=4)
    log_a = np.zeros(x.shape[:3])
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    H, G = x.shape[2], Bm.shape[2]
    for b in range(x.shape[0]):
        for h in range(H):
            g = h // (H // G)
            outer = Bm[b, :, g, :, None] * x[b, :, h, None, :]          # [T, N, P]
            states = h0[b, h][None] + np.cumsum(outer, axis=0)           # [T, N, P]
            want = np.einsum("tn,tnp->tp", Cm[b, :, g], states) + D[h] * x[b, :, h]
            _close(y[b, :, h], want, "a=1 y")
            _close(fin[b, h], h0[b, h] + Bm[b, :, g].T @ x[b, :, h], "a=1 final")


def pin_a_zero(orc):
    """a = 0 (encoded log a = -1e4, whose exp is exactly 0): the state forgets everything,
    y_t = (C_t . B_t) x_t + D x_t and final = B_{T-1} x_{T-1}^T (the Delta -> infinity limit
    A -> 0 of llms.blog "The Selection Mechanism")."""
    rng = np.random.default_rng(14)
    x, _, Bm, Cm, D, h0 = _problem(rng, nb=2, T=21, H=4, G=2, P=3, N=5)
    log_a = np.full(x.shape[:3], -1e4)
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    H, G = x.shape[2], Bm.shape[2]
    for b in range(x.shape[0]):
        for h in range(H):
            g = h // (H // G)
            cb = np.sum(Cm[b, :, g] * Bm[b, :, g], axis=1)             # [T]
            _close(y[b, :, h], (cb + D[h])[:, None] * x[b, :, h], "a=0 y")
            _close(fin[b, h], np.outer(Bm[b, -1, g], x[b, -1, h]), "a=0 final")


def pin_lti_convolution(orc):
    """Constant a, B, C (time-invariant): y = x * K with K_k = C^T B a^k (llms.blog, "The
    Duality of Inference and Training in Linear Time-Invariant SSMs"), checked per channel
    against numpy.convolve."""
    rng = np.random.default_rng(15)
    nb, T, H, G, P, N = 1, 64, 2, 1, 4, 6
    x = rng.standard_normal((nb, T, H, P))
    b_vec = rng.standard_normal(N)
    c_vec = rng.standard_normal(N)
    Bm = np.broadcast_to(b_vec, (nb, T, G, N)).copy()
    Cm = np.broadcast_to(c_vec, (nb, T, G, N)).copy()
    a_head = np.array([0.9, 0.6])
    log_a = np.broadcast_to(np.log(a_head), (nb, T, H)).copy()
    D = np.zeros(H)
    y, _ = orc.forward(x, log_a, Bm, Cm, D, None)
    for h in range(H):
        kernel = float(c_vec @ b_vec) * a_head[h] ** np.arange(T)
        for p in range(P):
            want = np.convolve(x[0, :, h, p], kernel)[:T]
            _close(y[0, :, h, p], want, "LTI convolution")


# --- structure ---------------------------------------------------------------------------
def _associative_prefix(pairs_a, pairs_b):
    """Inclusive prefix of (a_t, b_t) under (a_j, b_j) . (a_i, b_i) = (a_j a_i, a_j b_i + b_j)
    (llms.blog "Hardware-Aware Parallel Associative Scan"), evaluated by a Blelloch
    up-sweep / down-sweep tree rather than left to right.  a: [T, N], b: [T, N, P]."""
    T = pairs_a.shape[0]
    size = 1
    while size < T:
        size *= 2
    N, P = pairs_b.shape[1], pairs_b.shape[2]
    A = np.ones((size, N))
    Bv = np.zeros((size, N, P))
    A[:T], Bv[:T] = pairs_a, pairs_b

    def combine(later_a, later_b, earlier_a, earlier_b):
        return later_a * earlier_a, later_a[:, None] * earlier_b + later_b

    # up-sweep
    step = 1
    while step < size:
        for i in range(2 * step - 1, size, 2 * step):
            A[i], Bv[i] = combine(A[i], Bv[i], A[i - step], Bv[i - step])
        step *= 2
    total_a, total_b = A[size - 1].copy(), Bv[size - 1].copy()
    # down-sweep (exclusive), identity = (1, 0)
    A[size - 1], Bv[size - 1] = np.ones(N), np.zeros((N, P))
    step = size // 2
    while step >= 1:
        for i in range(2 * step - 1, size, 2 * step):
            left_a, left_b = A[i - step].copy(), Bv[i - step].copy()
            A[i - step], Bv[i - step] = A[i], Bv[i]
            A[i], Bv[i] = combine(left_a, left_b, A[i], Bv[i])
        step //= 2
    # inclusive = exclusive prefix combined with own element
    inc_b = np.empty((T, N, P))
    for t in range(T):
        _, inc_b[t] = combine(pairs_a[t], pairs_b[t], A[t], Bv[t])
    return inc_b, total_a, total_b


def pin_associative_scan(orc):
    """Every state h_t from a Blelloch-order scan of (A_t, B_t x_t^T) pairs; y_t = C_t^T h_t
    + D x_t and the final state must match the sequential oracle.  The initial state enters
    as a leading pair (0, h_0).  Scalar and diagonal decay."""
    rng = np.random.default_rng(16)
    for diag in (False, True):
        x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=1, T=23, H=2, G=1, P=3, N=4, diag=diag)
        y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
        for h in range(2):
            T, N = x.shape[1], Bm.shape[3]
            a = np.exp(log_a[0, :, h]) if diag else np.repeat(np.exp(log_a[0, :, h])[:, None], N, 1)
            pa = np.concatenate([np.zeros((1, N)), a])
            pb = np.concatenate([h0[0, h][None], Bm[0, :, 0, :, None] * x[0, :, h, None, :]])
            states, _, tot_b = _associative_prefix(pa, pb)
            states = states[1:]
            want_y = np.einsum("tn,tnp->tp", Cm[0, :, 0], states) + D[h] * x[0, :, h]
            _close(y[0, :, h], want_y, "associative scan y (diag=%s)" % diag)
            _close(fin[0, h], tot_b, "associative scan final (diag=%s)" % diag)


def pin_split_resume(orc):
    """Running T1 tokens, then T2 tokens from the returned state, equals running T1+T2."""
    rng = np.random.default_rng(17)
    for diag in (False, True):
        x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=2, T=30, H=4, G=2, P=3, N=4, diag=diag)
        y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
        t1 = 11
        ya, fa = orc.forward(x[:, :t1], log_a[:, :t1], Bm[:, :t1], Cm[:, :t1], D, h0)
        yb, fb = orc.forward(x[:, t1:], log_a[:, t1:], Bm[:, t1:], Cm[:, t1:], D, fa)
        _close(np.concatenate([ya, yb], axis=1), y, "split y")
        _close(fb, fin, "split final")


def pin_linearity(orc):
    """y and the final state are linear in (x, h_0) for fixed (log a, B, C, D=0)."""
    rng = np.random.default_rng(18)
    x1, log_a, Bm, Cm, _, h1 = _problem(rng, nb=1, T=25, H=2, G=1, P=4, N=3)
    x2 = rng.standard_normal(x1.shape)
    h2 = rng.standard_normal(h1.shape)
    D = np.zeros(x1.shape[2])
    al, be = 0.7, -1.3
    y1, f1 = orc.forward(x1, log_a, Bm, Cm, D, h1)
    y2, f2 = orc.forward(x2, log_a, Bm, Cm, D, h2)
    y3, f3 = orc.forward(al * x1 + be * x2, log_a, Bm, Cm, D, al * h1 + be * h2)
    _close(y3, al * y1 + be * y2, "linearity y")
    _close(f3, al * f1 + be * f2, "linearity final")


def pin_diag_equal_rates_is_scalar(orc):
    """A diagonal decay equal across state dimensions gives the scalar result."""
    rng = np.random.default_rng(19)
    x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=2, T=19, H=4, G=2, P=3, N=5)
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    log_a_d = np.repeat(log_a[..., None], Bm.shape[3], axis=-1)
    yd, fd = orc.forward(x, log_a_d, Bm, Cm, D, h0)
    _close(yd, y, "diag==scalar y", rtol=0.0)
    _close(fd, fin, "diag==scalar final", rtol=0.0)


def pin_groups_replicate(orc):
    """Sharing B, C by groups of heads (h uses group h // (H/G), llms.blog "Multi-Head State
    Space Layers") equals giving every head its own copy of its group's B, C."""
    rng = np.random.default_rng(20)
    x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=2, T=17, H=6, G=3, P=3, N=4)
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    rep = np.repeat(np.arange(3), 2)
    yr, fr = orc.forward(x, log_a, Bm[:, :, rep], Cm[:, :, rep], D, h0)
    _close(yr, y, "group replication y", rtol=0.0)
    _close(fr, fin, "group replication final", rtol=0.0)


def pin_head_decay_is_per_head(orc):
    """Each head reads its own decay: permuting heads (x, log a, D, h_0 together, with one
    group) permutes the outputs."""
    rng = np.random.default_rng(21)
    x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=1, T=15, H=4, G=1, P=3, N=4)
    perm = np.array([2, 0, 3, 1])
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    yp, fp = orc.forward(x[:, :, perm], log_a[:, :, perm], Bm, Cm, D[perm], h0[:, perm])
    _close(yp, y[:, :, perm], "head permutation y", rtol=0.0)
    _close(fp, fin[:, perm], "head permutation final", rtol=0.0)


# --- the discretisation front-end (oracle/discretize.py) ---------------------------------
# These pins take the oracle handle and the discretisation module (or a copy of it with a
# planted mistake).
def pin_softplus_values(orc, disc):
    """softplus where it has a closed form: ln 2 at 0, 1 at ln(e - 1), 2 at ln(e^2 - 1),
    v + e^-v (to 1e-16) at v = 40, e^v at v = -40, 0 far below and v far above."""
    e = np.e
    v = np.array([0.0, np.log(e - 1.0), np.log(e * e - 1.0), 40.0, -40.0, -800.0, 800.0])
    want = np.array([np.log(2.0), 1.0, 2.0, 40.0 + np.exp(-40.0), np.exp(-40.0), 0.0, 800.0])
    got = disc.softplus(v)
    assert np.all(np.abs(got - want) <= 1e-14 * np.maximum(1.0, np.abs(want)) + 1e-300), (got, want)
    assert abs(got[4] / want[4] - 1.0) < 1e-15  # the tiny value itself, not just |err| < 1e-14


def _dt_tensors(rng, nb, T, H, G, P, N):
    x = rng.standard_normal((nb, T, H, P))
    Bm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((nb, T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((nb, H, N, P))
    return x, Bm, Cm, D, h0


def pin_dt_one_token(orc, disc):
    """One token in closed form.  dt + dt_bias = ln(e^2 - 1), so Delta = softplus(.) = 2, and
    zero-order hold gives A-bar = exp(Delta A) = exp(-2 exp(A_log)) per head (per (head, state
    dim) for diagonal decay); A_log = ln 1.5 in head 0 (state dim 0) makes that e^-3.  Then
    h_1 = A-bar h_0 + 2 B x^T (B-bar = Delta B), or + B x^T without the input scale, and
    y = C . h_1 + D x with the raw x."""
    rng = np.random.default_rng(31)
    nb, H, G, P, N = 2, 3, 1, 2, 4
    x, Bm, Cm, D, h0 = _dt_tensors(rng, nb, 1, H, G, P, N)
    bias = np.array([0.25, -0.5, 1.0])
    dt = np.log(np.e ** 2 - 1.0) - np.broadcast_to(bias, (nb, 1, H))
    for diag in (False, True):
        A_log = rng.uniform(0.0, np.log(16.0), (H, N) if diag else (H,))
        A_log.flat[0] = np.log(1.5)
        for scale in (True, False):
            y, fin = disc.forward_dt(orc, x, dt, A_log, Bm, Cm, D, dt_bias=bias, scale_input=scale,
                                     init_state=h0, diag=diag)
            k = 2.0 if scale else 1.0
            for b in range(nb):
                for h in range(H):
                    abar = np.array([np.exp(-2.0 * np.exp(A_log[h, n] if diag else A_log[h])) for n in range(N)])
                    if h == 0:
                        assert abs(abar[0] - np.exp(-3.0)) < 1e-16
                    want_h = abar[:, None] * h0[b, h] + k * np.outer(Bm[b, 0, 0], x[b, 0, h])
                    _close(fin[b, h], want_h, "one token final (diag=%d scale=%d)" % (diag, scale), 1e-14)
                    _close(y[b, 0, h], Cm[b, 0, 0] @ want_h + D[h] * x[b, 0, h],
                           "one token y (diag=%d scale=%d)" % (diag, scale), 1e-14)


def pin_dt_limits(orc, disc):
    """The two limits of the selection mechanism.  Delta -> 0 (dt = -60): A-bar -> I and
    B-bar -> 0, so the state is kept and the tokens ignored: y_t = C_t . h_0 + D x_t and
    final = h_0.  Delta -> infinity (dt = 60, A_log = 0, so Delta = 60 up to e^-60): A-bar -> 0,
    so only the current token counts: y_t = 60 (C_t . B_t) x_t + D x_t and
    final = 60 B_{T-1} x_{T-1}^T."""
    rng = np.random.default_rng(32)
    nb, T, H, G, P, N = 2, 7, 4, 2, 3, 5
    x, Bm, Cm, D, h0 = _dt_tensors(rng, nb, T, H, G, P, N)
    A_log = rng.uniform(0.0, np.log(16.0), H)
    y, fin = disc.forward_dt(orc, x, np.full((nb, T, H), -60.0), A_log, Bm, Cm, D, init_state=h0)
    for b in range(nb):
        for h in range(H):
            g = h // (H // G)
            _close(y[b, :, h], Cm[b, :, g] @ h0[b, h] + D[h] * x[b, :, h], "Delta->0 y")
            _close(fin[b, h], h0[b, h], "Delta->0 final")
    y, fin = disc.forward_dt(orc, x, np.full((nb, T, H), 60.0), np.zeros(H), Bm, Cm, D, init_state=h0)
    for b in range(nb):
        for h in range(H):
            g = h // (H // G)
            cb = np.sum(Cm[b, :, g] * Bm[b, :, g], axis=1)
            _close(y[b, :, h], (60.0 * cb + D[h])[:, None] * x[b, :, h], "Delta->inf y")
            _close(fin[b, h], 60.0 * np.outer(Bm[b, -1, g], x[b, -1, h]), "Delta->inf final")


def pin_dt_diag_equal_rates_is_scalar(orc, disc):
    """A_log [H,N] whose columns are equal gives the scalar-decay result, bitwise in fp64."""
    rng = np.random.default_rng(33)
    nb, T, H, G, P, N = 2, 11, 4, 2, 3, 5
    x, Bm, Cm, D, h0 = _dt_tensors(rng, nb, T, H, G, P, N)
    dt = rng.standard_normal((nb, T, H)) - 2.0
    A_log = rng.uniform(0.0, np.log(16.0), H)
    bias = rng.standard_normal(H)
    ys, fs = disc.forward_dt(orc, x, dt, A_log, Bm, Cm, D, dt_bias=bias, init_state=h0)
    yd, fd = disc.forward_dt(orc, x, dt, np.repeat(A_log[:, None], N, axis=1), Bm, Cm, D, dt_bias=bias,
                             init_state=h0, diag=True)
    _close(yd, ys, "diag equal rates y", rtol=0.0)
    _close(fd, fs, "diag equal rates final", rtol=0.0)


DT_PINS = [pin_softplus_values, pin_dt_one_token, pin_dt_limits, pin_dt_diag_equal_rates_is_scalar]


ALL_PINS = [
    pin_handworked_scalar, pin_handworked_diag, pin_materialized_scalar, pin_materialized_diag,
    pin_a_one, pin_a_zero, pin_lti_convolution, pin_associative_scan, pin_split_resume,
    pin_linearity, pin_diag_equal_rates_is_scalar, pin_groups_replicate,
    pin_head_decay_is_per_head,
]
