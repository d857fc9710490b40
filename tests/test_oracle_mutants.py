"""Each planted mistake in a copy of the C oracle must be caught by at least one pin.

The mutants are textual edits of ``oracle/ssd_oracle.c`` compiled into a temporary
directory; the real oracle is never modified.  They cover the plausible slips: a dropped
term, a wrong sign, a wrong index, a transposed operand, a shifted time step."""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle.recurrence import SOURCE, Oracle, build
from pins import ALL_PINS

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
