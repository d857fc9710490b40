"""Pins of the oracle's packed variable-length forward (oracle/varlen.py), each checked against
something other than the per-sequence loop it runs: the recurrence over the whole packed token
axis with the decay forced to zero at every sequence start, and the closed form of the initial
state's contribution.  ``vl`` is the module under test (the real one or a planted mutant)."""
import numpy as np

from pins import _close


def _packed(rng, lens, H=3, G=1, P=4, N=5, diag=False):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = rng.standard_normal((T, H, P))
    Bm = rng.standard_normal((T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((T, G, N)) / np.sqrt(N)
    log_a = -np.log1p(np.exp(rng.standard_normal((T, H, N) if diag else (T, H))))
    D = rng.standard_normal(H)
    return cu, x, log_a, Bm, Cm, D


def pin_varlen_is_packed_run_with_resets(orc, vl):
    """Zero initial states: a packed batch equals one recurrence over the whole packed axis in
    which a_t = 0 (log a = -inf) at every sequence's first token, since then h_t = B_t x_t^T there,
    which is where a fresh sequence starts.  Each sequence's final state is that run's state at the
    sequence's last token, read as the final state of the run cut there.  Scalar and diagonal
    decay; lengths include 0, 1 and a long one."""
    rng = np.random.default_rng(91)
    for diag in (False, True):
        lens = [7, 0, 1, 23, 5, 0, 12]
        cu, x, log_a, Bm, Cm, D = _packed(rng, lens, diag=diag)
        y, fin = vl.forward_varlen(orc, x, log_a, Bm, Cm, cu, D)
        reset = log_a.copy()
        for i in range(len(lens)):
            if lens[i] > 0:
                reset[cu[i]] = -np.inf
        yr, _ = orc.forward(x[None], reset[None], Bm[None], Cm[None], D)
        _close(y, yr[0], "packed y (diag=%d)" % diag, rtol=1e-13)
        for i in range(len(lens)):
            e = int(cu[i + 1])
            if lens[i] == 0:
                _close(fin[i], np.zeros_like(fin[i]), "empty sequence %d final" % i, rtol=0.0)
                continue
            _, fr = orc.forward(x[None, :e], reset[None, :e], Bm[None, :e], Cm[None, :e], D)
            _close(fin[i], fr[0], "final of sequence %d (diag=%d)" % (i, diag), rtol=1e-13)


def pin_varlen_initial_states_closed_form(orc, vl):
    """With initial states h0_i, y and the finals move by the initial state's own term: for token t
    of sequence i, C_t^T (prod_{s = start_i .. t} a_s) h0_i (per state dim n for the diagonal
    decay), and the final by (prod over the whole sequence) h0_i.  An empty sequence returns h0_i."""
    rng = np.random.default_rng(92)
    for diag in (False, True):
        lens = [9, 0, 14, 1]
        H, G, P, N = 4, 2, 3, 5
        cu, x, log_a, Bm, Cm, D = _packed(rng, lens, H=H, G=G, P=P, N=N, diag=diag)
        h0 = rng.standard_normal((len(lens), H, N, P))
        y0, f0 = vl.forward_varlen(orc, x, log_a, Bm, Cm, cu, D)
        y1, f1 = vl.forward_varlen(orc, x, log_a, Bm, Cm, cu, D, init_states=h0)
        dy = np.zeros_like(y0)
        df = np.zeros_like(f0)
        for i in range(len(lens)):
            s, e = int(cu[i]), int(cu[i + 1])
            run = np.zeros((H, N))
            for t in range(s, e):
                run = run + (log_a[t][:, :] if diag else log_a[t][:, None])
                for h in range(H):
                    g = h // (H // G)
                    dy[t, h] = (Cm[t, g] * np.exp(run[h])) @ h0[i, h]
            df[i] = np.exp(run)[:, :, None] * h0[i]
        _close(y1 - y0, dy, "initial-state term of y (diag=%d)" % diag, rtol=1e-12)
        _close(f1 - f0, df, "initial-state term of the finals (diag=%d)" % diag, rtol=1e-12)


VARLEN_PINS = [pin_varlen_is_packed_run_with_resets, pin_varlen_initial_states_closed_form]


def pin_varlen_backward_finite_differences(orc, vl, adj):
    """backward_varlen against central differences (step 1e-6) of <dy, y> + <dfinal, finals> from
    forward_varlen, along a random direction in each of x, log a, B, C, D and the initial states;
    scalar and diagonal decay, lengths 0, 1 and longer."""
    rng = np.random.default_rng(93)
    for diag in (False, True):
        lens = [6, 0, 1, 11]
        H, G, P, N = 4, 2, 3, 5
        cu, x, log_a, Bm, Cm, D = _packed(rng, lens, H=H, G=G, P=P, N=N, diag=diag)
        h0 = rng.standard_normal((len(lens), H, N, P))
        dy = rng.standard_normal(x.shape)
        dfin = rng.standard_normal(h0.shape)
        inp = dict(x=x, log_a=log_a, Bm=Bm, Cm=Cm, D=D, init=h0)

        def loss(d):
            y, fin = vl.forward_varlen(orc, d["x"], d["log_a"], d["Bm"], d["Cm"], cu, d["D"], d["init"])
            return float(np.sum(dy * y) + np.sum(dfin * fin))

        g = vl.backward_varlen(adj, x, log_a, Bm, Cm, cu, D, h0, dy, dfin)
        names = dict(x="dx", log_a="dlog_a", Bm="dB", Cm="dC", D="dD", init="dinit")
        eps = 1e-6
        for name, gname in names.items():
            v = rng.standard_normal(np.shape(inp[name]))
            fd = (loss(dict(inp, **{name: inp[name] + eps * v})) - loss(dict(inp, **{name: inp[name] - eps * v}))) \
                / (2 * eps)
            an = float(np.sum(g[gname] * v))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), "%s (diag=%d): fd %.12g adjoint %.12g" % (
                gname, diag, fd, an)
