"""The oracle's packed variable-length forward against its pins, and planted mistakes in it
that the pins must catch."""
import importlib.util
import os
import tempfile

import numpy as np
import pytest

import oracle
import oracle.backward
import oracle.varlen
from pins_varlen import VARLEN_PINS, pin_varlen_backward_finite_differences


@pytest.fixture(scope="module")
def orc():
    return oracle.default_oracle()


@pytest.mark.parametrize("pin", VARLEN_PINS, ids=lambda p: p.__name__)
def test_varlen_pin(orc, pin):
    pin(orc, oracle.varlen)


def test_cu_seqlens_checked():
    for bad in ([1, 4], [0, 3, 2, 4], [0, 2, 5], [[0, 4]], []):
        with pytest.raises(ValueError):
            oracle.varlen.check_cu_seqlens(bad, 4)


MUTANTS = {
    "state_carried_over": ("init = None if init_states is None else np.asarray(init_states, dtype=np.float64)[i:i + 1]",
                           "init = (None if init_states is None else np.asarray(init_states, dtype=np.float64)[i:i + 1]) "
                           "if i == 0 or finals is None else finals[i - 1:i]"),
    "start_off_by_one": ("s, e = int(cu[i]), int(cu[i + 1])", "s, e = int(cu[i]) + (1 if cu[i + 1] > cu[i] + 1 else 0), int(cu[i + 1])"),
    "first_init_for_all": ("np.asarray(init_states, dtype=np.float64)[i:i + 1]", "np.asarray(init_states, dtype=np.float64)[0:1]"),
    "empty_keeps_zero": ("            if want_final and init is not None:\n                finals[i] = init[0]\n",
                         "            pass\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_varlen_mutant_is_caught(orc, name):
    before, after = MUTANTS[name]
    with open(oracle.varlen.__file__) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "varlen_%s.py" % name)
        with open(path, "w") as f:
            f.write(src.replace(before, after))
        spec = importlib.util.spec_from_file_location("varlen_%s" % name, path)
        mutant = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mutant)
        caught = []
        for pin in VARLEN_PINS:
            try:
                pin(orc, mutant)
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name


def test_varlen_backward_pin(orc):
    pin_varlen_backward_finite_differences(orc, oracle.varlen, oracle.backward.default_adjoint())


BWD_MUTANTS = {
    "dD_of_last_sequence_only": ('        out["dD"] += g["dD"]', '        out["dD"] = g["dD"].copy()'),
    "empty_drops_dfinal": ('            if fin is not None:\n                out["dinit"][i] = fin[0]\n', '            pass\n'),
    "dfinal_of_first_for_all": ('np.asarray(dfinal, dtype=np.float64)[i:i + 1]', 'np.asarray(dfinal, dtype=np.float64)[0:1]'),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_varlen_backward_mutant_is_caught(orc, name):
    before, after = BWD_MUTANTS[name]
    with open(oracle.varlen.__file__) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation site for %s must occur exactly once" % name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "varlen_bwd_%s.py" % name)
        with open(path, "w") as f:
            f.write(src.replace(before, after))
        spec = importlib.util.spec_from_file_location("varlen_bwd_%s" % name, path)
        mutant = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mutant)
        with pytest.raises(AssertionError):
            pin_varlen_backward_finite_differences(orc, mutant, oracle.backward.default_adjoint())
