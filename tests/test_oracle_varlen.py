"""The oracle's packed variable-length forward against its pins, and planted mistakes in it
that the pins must catch."""
import importlib.util
import os
import tempfile

import numpy as np
import pytest

import oracle
import oracle.varlen
from pins_varlen import VARLEN_PINS


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
