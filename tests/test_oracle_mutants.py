"""Each planted mistake in a copy of the C oracle must be caught by at least one pin.

The mutants are textual edits of ``oracle/ssd_oracle.c`` compiled into a temporary
directory; the real oracle is never modified.  They cover the plausible slips: a dropped
term, a wrong sign, a wrong index, a transposed operand, a shifted time step."""
import os
import shutil
import tempfile

import importlib.util

import pytest

import oracle
import oracle.discretize
from oracle.recurrence import SOURCE, Oracle, build
from pins import ALL_PINS, DT_PINS

MUTANTS = {
    "decay_dropped": ("decay[n] * state[n * P + p] + bt[n] * xt[p]",
                      "state[n * P + p] + bt[n] * xt[p]"),
    "decay_after_input": ("decay[n] * state[n * P + p] + bt[n] * xt[p]",
                          "decay[n] * (state[n * P + p] + bt[n] * xt[p])"),
    "decay_sign": ("exp(log_a[row * N + n]) : exp(log_a[row])",
                   "exp(-log_a[row * N + n]) : exp(-log_a[row])"),
    "diag_index": ("exp(log_a[row * N + n])", "exp(log_a[row * N])"),
    "skip_dropped": ("double acc = D ? D[hd] * xt[p] : 0.0;", "double acc = 0.0;"),
    "readout_uses_B": ("acc += ct[n] * state[n * P + p];", "acc += bt[n] * state[n * P + p];"),
    "readout_transposed": ("acc += ct[n] * state[n * P + p];",
                           "acc += ct[n] * state[(p * N + n) % (N * P)];"),
    "input_uses_C": ("+ bt[n] * xt[p];", "+ ct[n] * xt[p];"),
    "init_ignored": ("init_state ? init_state[((b * H + hd) * N + n) * P + p] : 0.0",
                     "0.0"),
    "wrong_group": ("const int64_t g = hd / heads_per_group;", "const int64_t g = hd % G;"),
    "skip_previous_token": ("double acc = D ? D[hd] * xt[p] : 0.0;",
                            "double acc = D ? D[hd] * (t > 0 ? xt[p - H * P] : xt[p]) : 0.0;"),
    "final_before_last_step": ("for (int64_t t = 0; t < T; ++t) {",
                               "for (int64_t t = 0; t < T; ++t) { if (t == T - 1 && final_state) break;"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="ssd_oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    before, after = MUTANTS[name]
    with open(SOURCE) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    path = os.path.join(workdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    lib = build(path, os.path.join(workdir, "lib_%s.so" % name))
    mutant = Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name


# planted mistakes in a copy of the discretisation front-end (oracle/discretize.py)
DT_MUTANTS = {
    "softplus_is_exp": ("np.logaddexp(0.0, np.asarray(v, dtype=np.float64))",
                        "np.exp(np.asarray(v, dtype=np.float64))"),
    "softplus_is_identity": ("np.logaddexp(0.0, np.asarray(v, dtype=np.float64))",
                             "np.asarray(v, dtype=np.float64)"),
    "A_positive": ("A = -np.exp(A_log)", "A = np.exp(A_log)"),
    "A_is_A_log": ("A = -np.exp(A_log)", "A = -A_log"),
    "bias_dropped": ("v = dt if dt_bias is None else dt + np.asarray(dt_bias, dtype=np.float64)[None, None, :]",
                     "v = dt"),
    "bias_subtracted": ("else dt + np.asarray(dt_bias", "else dt - np.asarray(dt_bias"),
    "delta_not_in_decay": ("log_a = delta * A[None, None, :]", "log_a = A[None, None, :] + 0 * delta"),
    "diag_delta_not_in_decay": ("log_a = delta[..., None] * A[None, None, :, :]",
                                "log_a = 0 * delta[..., None] + A[None, None, :, :]"),
    "input_not_scaled": ("xin = x * delta[..., None] if scale_input else x", "xin = x"),
    "input_always_scaled": ("xin = x * delta[..., None] if scale_input else x", "xin = x * delta[..., None]"),
    "skip_on_scaled_input": ("[None, None, :, None] * x\n", "[None, None, :, None] * xin\n"),
    "skip_dropped": ("        y = y + np.asarray(D, dtype=np.float64)[None, None, :, None] * x\n",
                     "        y = y\n"),
    "diag_rates_of_first_dim": ("A[None, None, :, :]", "np.repeat(A[:, :1], A.shape[1], axis=1)[None, None]"),
    "diag_rates_of_first_head": ("A[None, None, :, :]", "np.repeat(A[:1, :], A.shape[0], axis=0)[None, None]"),
}


@pytest.fixture(scope="module")
def real_oracle():
    return oracle.default_oracle()


@pytest.mark.parametrize("name", sorted(DT_MUTANTS))
def test_discretization_mutant_is_caught(workdir, real_oracle, name):
    before, after = DT_MUTANTS[name]
    src_path = oracle.discretize.__file__
    with open(src_path) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    path = os.path.join(workdir, "discretize_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    spec = importlib.util.spec_from_file_location("discretize_%s" % name, path)
    mutant = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mutant)
    caught = []
    for pin in DT_PINS:
        try:
            pin(real_oracle, mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
