"""The oracle's backward pass (oracle/backward.py) against its pins, and planted mistakes in
copies of its C source, each of which some pin must catch."""
import os
import shutil
import tempfile

import pytest

import importlib.util

import oracle
import oracle.backward as bwd
import oracle.discretize
from pins_bwd import BWD_DT_PINS, BWD_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default_oracle()


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(orc, pin):
    pin(orc, bwd.default_adjoint())


MUTANTS = {
    "skip_dropped_from_dx": ("double acc = D ? D[hd] * dyt[p] : 0.0;", "double acc = 0.0;"),
    "readout_after_dx": ("Gs[n * P + p] += ct[n] * dyt[p];", "Gs[n * P + p] += 0.0 * ct[n] * dyt[p];"),
    "dx_uses_C": ("acc += Gs[n * P + p] * bt[n];", "acc += Gs[n * P + p] * ct[n];"),
    "dB_uses_dy": ("gb += Gs[n * P + p] * xt[p];", "gb += Gs[n * P + p] * dyt[p];"),
    "dC_uses_prev_state": ("gc += ht[n * P + p] * dyt[p];", "gc += hprev[n * P + p] * dyt[p];"),
    "dloga_uses_current_state": ("acc += Gs[i] * hprev[i];", "acc += Gs[i] * ht[i];"),
    "dloga_without_a": ("dlog_a[row] = a[0] * acc;", "dlog_a[row] = acc;"),
    "diag_dloga_summed_over_n": ("dlog_a[row * N + n] = a[n] * acc;", "dlog_a[row * N + n] = a[0] * acc;"),
    "G_not_decayed": ("for (int64_t p = 0; p < P; ++p) Gs[n * P + p] *= a[n];",
                      "for (int64_t p = 0; p < P; ++p) Gs[n * P + p] *= 1.0;"),
    "dfinal_ignored": ("Gs[i] = dfinal ? dfinal[(b * H + hd) * N * P + i] : 0.0;", "Gs[i] = 0.0;"),
    "dD_wrong_operand": ("dDh += dyt[p] * xt[p];", "dDh += dyt[p] * dyt[p];"),
    "init_ignored": ("hs[i] = init_state ? init_state[(b * H + hd) * N * P + i] : 0.0;", "hs[i] = 0.0;"),
    "dB_last_head_only": ("dbt[n] += gb;", "dbt[n] = gb;"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="ssd_adjoint_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(orc, workdir, name):
    before, after = MUTANTS[name]
    with open(bwd.SOURCE) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    path = os.path.join(workdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    mutant = bwd.Adjoint(bwd.build(path, os.path.join(workdir, "lib_%s.so" % name)))
    caught = []
    for pin in BWD_PINS:
        try:
            pin(orc, mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name


@pytest.mark.parametrize("pin", BWD_DT_PINS, ids=lambda p: p.__name__)
def test_backward_dt_pin(orc, pin):
    pin(orc, bwd.default_adjoint(), oracle.discretize)


# planted mistakes in a copy of the discretisation module's chain rule
DT_MUTANTS = {
    "sigmoid_is_softplus": ("ddt = ddelta * sigmoid(u)", "ddt = ddelta * softplus(u)"),
    "A_sign": ("ddelta = g[\"dlog_a\"] * A[None, None, :]", "ddelta = -g[\"dlog_a\"] * A[None, None, :]"),
    "scale_term_dropped": ("ddelta = ddelta + np.sum(dxin * x, axis=-1)", "ddelta = ddelta"),
    "dx_not_scaled": ("dx = dxin * delta[..., None] if scale_input else dxin.copy()", "dx = dxin.copy()"),
    "dA_log_uses_delta": ("np.sum(g[\"dlog_a\"] * log_a, axis=(0, 1))", "np.sum(g[\"dlog_a\"] * delta, axis=(0, 1))"),
    "bias_not_in_sigmoid": ("u = u + np.asarray(dt_bias, dtype=np.float64)[None, None, :]", "u = u"),
    "dD_on_scaled_input": ("dD=np.einsum(\"bthp,bthp->h\", dy, x)", "dD=np.einsum(\"bthp,bthp->h\", dy, xin)"),
    "diag_rates_summed_first": ("ddelta = np.einsum(\"bthn,hn->bth\", g[\"dlog_a\"], A)",
                                "ddelta = np.sum(g[\"dlog_a\"], axis=-1) * np.mean(A, axis=-1)[None, None, :]"),
    "diag_one_rate": ("ddelta = np.einsum(\"bthn,hn->bth\", g[\"dlog_a\"], A)",
                      "ddelta = np.sum(g[\"dlog_a\"], axis=-1) * A[None, None, :, 0]"),
}


@pytest.mark.parametrize("name", sorted(DT_MUTANTS))
def test_backward_dt_mutant_is_caught(orc, workdir, name):
    before, after = DT_MUTANTS[name]
    with open(oracle.discretize.__file__) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    path = os.path.join(workdir, "disc_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    spec = importlib.util.spec_from_file_location("disc_%s" % name, path)
    mutant = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mutant)
    caught = []
    for pin in BWD_DT_PINS:
        try:
            pin(orc, bwd.default_adjoint(), mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
