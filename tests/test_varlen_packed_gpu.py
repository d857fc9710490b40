"""Packed variable-length batches with no per-sequence states (init_state and final_state both
NULL): the fast path then walks the whole packed token axis as one sequence, segmented like a
long batched sequence, with the recurrence restarted at every sequence's first token.  Every
output is compared with the oracle's per-sequence recurrence (oracle.varlen.forward_varlen) on
the same seeded inputs, over all tokens and sequence by sequence; bounds as for ssd_forward
(relative L2 <= 2e-2 for bf16).  Cases mix empty, one-token and chunk-crossing sequences with
sequences long enough to span several segments (so the segment-state chain both restarts and
carries across segment boundaries), grouped heads, chunks 64, 128 and 256, the discretisation
front-end, a sequence longer than the length bound (its tokens past the bound, and tokens after
the last offset, are never written), and a NaN-filled workspace."""
import numpy as np
import pytest
import torch

import oracle
import oracle.discretize
import oracle.varlen
import ssd_inputs
import ssd_chunked_scan_02_amd as ssd
from gpu_helpers import announce, rel_l2, TOL, OUT_ROUNDOFF

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64


def _mix(nseq, total, seed, extra=()):
    """A seeded log-normal length mix with some empty and one-token sequences spliced in."""
    lengths = ssd_inputs.packed_lengths(nseq, total, seed, spread=1.5)
    for i in range(0, len(lengths), 7):
        lengths[i] = 0 if (i // 7) % 2 == 0 else 1
    return lengths + list(extra)


CASES = [
    ("mamba2_layer", dict(nheads=4), 128, _mix(120, 4000, 5, extra=(2100, 1)), "q128-short-and-long"),
    ("gqa_decode", dict(nheads=8, ngroups=2, decode_steps=0), 64, _mix(300, 3000, 6), "q64-gqa-many-short"),
    ("mamba2_layer", dict(nheads=2, dstate=64), 256, [5000, 3, 0, 2000, 17], "q256-n64-long-chains"),
    ("mamba2_layer", dict(nheads=8), 128, [1] * 600 + [0, 129, 128, 127], "q128-one-token-runs"),
    # no skip term: y is the SSD part alone, under the plain bound
    ("mamba2_layer", dict(nheads=4, skip=False), 128, _mix(60, 3000, 7, extra=(1500,)), "q128-no-skip"),
]


def _ssd_part_error(yg, yr, x, D, dtype):
    """relL2 of y - D x (the SSD part) and its bound: the bf16 output rounding is relative to the
    whole of y, which the skip term may dominate."""
    skip = 0.0 if D is None else D[None, :, None] * x
    e = rel_l2(yg - skip, yr - skip)
    ssd_norm = float(np.linalg.norm((yr - skip).ravel()))
    bound = TOL[dtype] + (OUT_ROUNDOFF[dtype] * float(np.linalg.norm(yr.ravel())) / ssd_norm if ssd_norm > 0 else 0)
    return e, bound


class _Events:
    """hipEvent_t handles for one profiled call (the launch count comes back with them)."""

    def __enter__(self):
        from bench import HipEvents
        self.ev = HipEvents()
        self.handles = [self.ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)]
        return self.handles

    def __exit__(self, *exc):
        torch.cuda.synchronize()
        for h in self.handles:
            self.ev.destroy(h)


def _check_per_sequence(y, yr, cu, lengths, x, D, dtype):
    """Every nonempty sequence by itself, on its SSD part under _ssd_part_error's bound: a short
    sequence's y can nearly cancel (a one-token sequence has y = (C.B + D) x, and C.B close to -D
    leaves the bf16 rounding of the score C.B as a large part of what remains)."""
    for i, n in enumerate(lengths):
        s, e = int(cu[i]), int(cu[i + 1])
        if n > 0:
            err, bound = _ssd_part_error(y[s:e], yr[s:e], x[s:e], D, dtype)
            assert err <= bound, "sequence %d: SSD part %.3e, bound %.3e" % (i, err, bound)


@pytest.mark.parametrize("name,over,chunk,lengths,label", CASES, ids=[c[4] for c in CASES])
def test_packed_as_one_matches_oracle(name, over, chunk, lengths, label):
    cfg = ssd_inputs.config(name, init=False, **over)
    announce("packed-as-one %s: %d sequences, %d tokens, chunk %d" % (label, len(lengths), sum(lengths), chunk))
    p = ssd_inputs.packed_inputs(cfg, lengths, 61)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    # (a NaN-filled workspace: nothing may read a part of it before writing it)
    dims = ssd.varlen_dims(g["x"], g["log_a"], g["B"], len(lengths), p["max_seqlen"])
    ws = torch.full((ssd.ssd_forward_varlen_workspace_bytes(dims, chunk) // 4 + 1,), float("nan"),
                    dtype=torch.float32, device="cuda")
    with _Events() as events:
        y, fin, launches = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"],
                                                  p["max_seqlen"], g.get("D"), chunk=chunk, workspace=ws, events=events)
    assert fin is None
    # the prep (which also marks the tokens) and the walk, and the segment states when segmented
    assert launches in (2, 3), launches
    yr, _ = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                         f64(p["C"]), p["cu_seqlens"].numpy(), f64(p.get("D")), None, want_final=False)
    tol = TOL[cfg["dtype"]]
    yg = y.double().cpu().numpy()
    ey = rel_l2(yg, yr)
    es, bound = _ssd_part_error(yg, yr, f64(p["x"]), f64(p.get("D")), cfg["dtype"])
    announce("packed-as-one %s: y %.2e, SSD part %.2e (bound %.2e), %d launches" % (label, ey, es, bound, launches))
    assert ey <= tol and es <= bound, (ey, es, bound)
    _check_per_sequence(yg, yr, p["cu_seqlens"].numpy(), lengths, f64(p["x"]), f64(p.get("D")), cfg["dtype"])


def test_packed_as_one_front_end_matches_oracle():
    """ssd_forward_dt_varlen with no states: the oracle's discretisation, then its per-sequence
    recurrence on the scaled input, and D x on the raw x."""
    cfg = ssd_inputs.config("mamba2_layer", nheads=4, init=False)
    lengths = _mix(90, 3000, 8, extra=(1500,))
    announce("packed-as-one dt: %d sequences, %d tokens" % (len(lengths), sum(lengths)))
    p = ssd_inputs.packed_inputs(cfg, lengths, 67)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 68)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    with _Events() as events:
        y, fin, launches = ssd.ssd_forward_dt_varlen(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g["cu_seqlens"],
                                                     p["max_seqlen"], g.get("D"), dt_bias=bias.cuda(),
                                                     scale_input=True, chunk=128, events=events)
    assert fin is None and launches in (2, 3), launches
    delta, la = oracle.discretize.discretize(f64(p["dt"])[None], f64(p["A_log"]), f64(bias), False)
    x = f64(p["x"])
    yr, _ = oracle.varlen.forward_varlen(oracle.default_oracle(), x * delta[0][..., None], la[0], f64(p["B"]),
                                         f64(p["C"]), p["cu_seqlens"].numpy(), None, None, want_final=False)
    yr = yr + f64(p["D"])[None, :, None] * x
    tol = TOL[cfg["dtype"]]
    yg = y.double().cpu().numpy()
    ey = rel_l2(yg, yr)
    announce("packed-as-one dt: y %.2e (tol %.0e)" % (ey, tol))
    assert ey <= tol, ey
    _check_per_sequence(yg, yr, p["cu_seqlens"].numpy(), lengths, x, f64(p["D"]), cfg["dtype"])


def test_packed_as_one_length_bound_and_uncovered_tokens():
    """A sequence longer than the length bound is walked to its first `bound` tokens only, and its
    tokens past the bound are not written; neither are the tokens after the last offset.  The other
    sequences are unaffected."""
    cfg = ssd_inputs.config("mamba2_layer", nheads=8, init=False)
    lengths = [3] * 300 + [50, 300, 40, 0, 170, 7]
    bound = 200
    tail = 33  # tokens after the last offset
    announce("packed-as-one bound %d, lengths %s, %d uncovered tokens" % (bound, lengths, tail))
    p = ssd_inputs.packed_inputs(cfg, lengths + [tail], 71)
    cu = p["cu_seqlens"][:-1].clone()  # the last sequence dropped: its tokens are past every offset
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    y = torch.full_like(g["x"], float("nan"))
    with _Events() as events:
        _, _, launches = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], cu.cuda(), bound, g.get("D"),
                                                chunk=128, y=y, events=events)
    assert launches in (2, 3), launches
    yg = y.double().cpu().numpy()
    tol = TOL[cfg["dtype"]]
    x, la, Bm, Cm, D = f64(p["x"]), f64(p["log_a"]), f64(p["B"]), f64(p["C"]), f64(p["D"])
    orc = oracle.default_oracle()
    for i, n in enumerate(lengths):
        s = int(cu[i])
        e = s + min(n, bound)
        if n > 0:
            yr, _ = orc.forward(x[None, s:e], la[None, s:e], Bm[None, s:e], Cm[None, s:e], D, None, False)
            assert rel_l2(yg[s:e], yr[0]) <= tol, "sequence %d" % i
        # past the bound: untouched
        assert np.isnan(yg[e:s + n]).all(), "sequence %d tokens past the bound were written" % i
    assert np.isnan(yg[int(cu[-1]):]).all(), "tokens after the last offset were written"


def test_packed_as_one_many_sequences_full_size():
    """The 16 384 tokens of the Mamba-2 layer shape (24 heads) packed as 1024 sequences of a
    log-normal length mix, as the packed benchmark runs them; sampled sequences and the whole y."""
    cfg = ssd_inputs.config("mamba2_layer", init=False)
    lengths = ssd_inputs.packed_lengths(1024, cfg["batch"] * cfg["seqlen"], 9)
    announce("packed-as-one full size: 1024 sequences, %d tokens" % sum(lengths))
    p = ssd_inputs.packed_inputs(cfg, lengths, 73)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    with _Events() as events:
        y, _, launches = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"],
                                                p["max_seqlen"], g.get("D"), chunk=cfg["chunk"], events=events)
    assert launches == 3, launches
    yr, _ = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                         f64(p["C"]), p["cu_seqlens"].numpy(), f64(p["D"]), None, want_final=False)
    tol = TOL[cfg["dtype"]]
    yg = y.double().cpu().numpy()
    ey = rel_l2(yg, yr)
    es, bound = _ssd_part_error(yg, yr, f64(p["x"]), f64(p["D"]), cfg["dtype"])
    announce("packed-as-one full size: y %.2e, SSD part %.2e (bound %.2e)" % (ey, es, bound))
    assert ey <= tol and es <= bound, (ey, es, bound)
    _check_per_sequence(yg, yr, p["cu_seqlens"].numpy(), lengths, f64(p["x"]), f64(p["D"]), cfg["dtype"])


def test_packed_as_one_more_sequences_than_prep_marks():
    """5000 sequences of 0-9 tokens (more offsets than the prep kernel stages in LDS): the token
    flags come from a marking launch of their own; every sequence against the oracle."""
    cfg = ssd_inputs.config("mamba2_layer", nheads=2, init=False)
    rng = np.random.default_rng(83)
    lengths = [int(v) for v in rng.integers(0, 10, size=5000)]
    announce("packed-as-one, marking launch: %d sequences, %d tokens" % (len(lengths), sum(lengths)))
    p = ssd_inputs.packed_inputs(cfg, lengths, 79)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    with _Events() as events:
        y, _, launches = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"],
                                                p["max_seqlen"], g.get("D"), chunk=128, events=events)
    # the marking, the prep and the walk, and the segment states when segmented
    assert launches in (3, 4), launches
    yr, _ = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                         f64(p["C"]), p["cu_seqlens"].numpy(), f64(p["D"]), None, want_final=False)
    tol = TOL[cfg["dtype"]]
    yg = y.double().cpu().numpy()
    ey = rel_l2(yg, yr)
    es, bound = _ssd_part_error(yg, yr, f64(p["x"]), f64(p["D"]), cfg["dtype"])
    announce("packed-as-one, marking launch: y %.2e, SSD part %.2e (bound %.2e), %d launches" % (ey, es, bound, launches))
    assert ey <= tol and es <= bound, (ey, es, bound)
    _check_per_sequence(yg, yr, p["cu_seqlens"].numpy(), lengths, f64(p["x"]), f64(p["D"]), cfg["dtype"])
