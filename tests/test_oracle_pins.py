"""The CPU oracle against its pins (hand-worked examples, the matrix form, closed forms,
the LTI convolution, associative-scan order, split/resume, linearity, group sharing, the
discretisation front-end), and
the chunked fp64 model against the oracle for many chunk lengths."""
import numpy as np
import pytest

import oracle
import oracle.discretize
from pins import ALL_PINS, DT_PINS, _problem, _close


@pytest.fixture(scope="module")
def orc():
    return oracle.default_oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", DT_PINS, ids=lambda p: p.__name__)
def test_discretization_pin(orc, pin):
    pin(orc, oracle.discretize)


@pytest.mark.parametrize("diag", [False, True])
@pytest.mark.parametrize("chunk", [1, 5, 16, 32, 64, 100, 256])
def test_chunked_model_matches_recurrence(orc, diag, chunk):
    """Chunk-size invariance of the two-algorithm form (aiwiki "State Space Duality", "Two
    algorithms for one operator": where the chunk boundaries fall changes only which pairs the
    quadratic form covers and which the state carries, not the result), including a last chunk
    shorter than the others."""
    rng = np.random.default_rng(100 + chunk)
    prob = _problem(rng, nb=2, T=100, H=4, G=2, P=5, N=6, diag=diag, decay_scale=3.0)
    y, fin = orc.forward(*prob)
    yc, fc = oracle.chunked_forward(*prob, chunk=chunk)
    _close(yc, y, "chunked y", rtol=1e-11)
    _close(fc, fin, "chunked final", rtol=1e-11)


def test_oracle_empty_sequence(orc):
    """T = 0: no outputs, the final state is the initial state."""
    rng = np.random.default_rng(5)
    x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=2, T=0, H=2, G=1, P=3, N=4)
    y, fin = orc.forward(x, log_a, Bm, Cm, D, h0)
    assert y.shape == (2, 0, 2, 3)
    assert np.array_equal(fin, h0)


def test_oracle_threads_do_not_change_result(orc):
    rng = np.random.default_rng(6)
    prob = _problem(rng, nb=3, T=50, H=4, G=2, P=4, N=5)
    y1, f1 = orc.forward(*prob, nthreads=1)
    y4, f4 = orc.forward(*prob, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


@pytest.mark.parametrize("diag", [False, True])
@pytest.mark.parametrize("chunk", [7, 32])
def test_chunked_model_states_are_the_recurrence_states(orc, diag, chunk):
    """The states the chunked model carries between chunks (the H_{k-1} that enters chunk k) are
    the recurrence's state after the first k chunk-lengths of tokens: the oracle run on that
    prefix alone, from the same initial state, ends in it (the state passing of llms.blog "The
    Chunk-Wise SSD Algorithm").  Chunk 0 enters with the initial state itself."""
    rng = np.random.default_rng(300 + chunk)
    x, log_a, Bm, Cm, D, h0 = _problem(rng, nb=2, T=90, H=3, G=1, P=4, N=5, diag=diag, decay_scale=2.0)
    _, fin, prev = oracle.chunked_forward(x, log_a, Bm, Cm, D, h0, chunk=chunk, return_states=True)
    nchunks = -(-x.shape[1] // chunk)
    assert prev.shape[2] == nchunks
    _close(prev[:, :, 0], h0, "state entering chunk 0", rtol=0.0)
    for k in range(1, nchunks):
        t = k * chunk
        _, fk = orc.forward(x[:, :t], log_a[:, :t], Bm[:, :t], Cm[:, :t], D, h0)
        _close(prev[:, :, k], fk, "state entering chunk %d" % k, rtol=1e-11)
