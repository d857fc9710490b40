"""ssd_forward_varlen (packed variable-length batches) against the oracle's per-sequence
recurrence (oracle.varlen.forward_varlen), element by element on the same seeded inputs, on each
path: the bf16 fast path (chunks 64 and 128, grouped heads), the pipelined diagonal walk, and the
generic scalar and diagonal walks (fp32, and bf16 with a head dim off the fast path).  Lengths mix
empty, one-token, chunk-multiple and ragged sequences.  Bounds as for ssd_forward: relative L2
<= 1e-5 for fp32 inputs, <= 2e-2 for bf16, on y and on the final states."""
import numpy as np
import pytest
import torch

import oracle
import oracle.backward
import oracle.discretize
import oracle.varlen
import ssd_inputs
import ssd_chunked_scan_02_amd as ssd
from gpu_helpers import announce, rel_l2, TOL

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64

CASES = [
    ("mamba2_layer", dict(nheads=4, init=True), 128, [300, 1, 0, 129, 1000, 128, 57], "fast-q128"),
    ("gqa_decode", dict(nheads=8, ngroups=2, init=True, decode_steps=0), 64, [64, 700, 0, 3, 250], "fast-q64-gqa"),
    ("mamba2_layer", dict(nheads=2, dstate=64, init=False), 256, [1500, 255, 2], "fast-q256-n64"),
    ("diag_multiscale", dict(nheads=3, init=True), 64, [200, 0, 64, 1, 517], "diag-pipe"),
    ("diag_multiscale", dict(nheads=2, dstate=32, headdim=32, init=True, a_log="rand_hn"), 64, [100, 333, 7],
     "diag-pipe-32"),
    ("tiny_fp32", dict(nheads=3, skip=True, init=True), 64, [90, 0, 257, 64, 1], "generic-fp32"),
    ("mamba2_layer", dict(nheads=2, headdim=32, init=True), 128, [130, 400, 5], "generic-bf16-p32"),
    ("diag_multiscale", dict(nheads=2, dstate=16, headdim=32, dtype="fp32", init=True, a_log="rand_hn"), 32,
     [77, 0, 140], "generic-diag-fp32"),
]


def _run(name, over, chunk, lengths, label, seed=41):
    cfg = ssd_inputs.config(name, **over)
    announce("varlen %s lengths=%s chunk=%d" % (label, lengths, chunk))
    p = ssd_inputs.packed_inputs(cfg, lengths, seed)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    y, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"], p["max_seqlen"],
                                       g.get("D"), chunk=chunk, init_state=g.get("init_state"), final_state=True)
    torch.cuda.synchronize()
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                          f64(p["C"]), p["cu_seqlens"].numpy(), f64(p.get("D")),
                                          f64(p.get("init_state")))
    tol = TOL[cfg["dtype"]]
    ey = rel_l2(y.double().cpu().numpy(), yr) if yr.size else 0.0
    ef = rel_l2(fin.double().cpu().numpy(), fr)
    announce("varlen %s: y %.2e final %.2e (tol %.0e)" % (label, ey, ef, tol))
    assert ey <= tol and ef <= tol, (ey, ef)
    # each sequence on its own too: no sequence may hide another's error
    for i, n in enumerate(lengths):
        s, e = int(p["cu_seqlens"][i]), int(p["cu_seqlens"][i + 1])
        if n > 0:
            assert rel_l2(y[s:e].double().cpu().numpy(), yr[s:e]) <= tol, "sequence %d y" % i
        assert rel_l2(fin[i].double().cpu().numpy(), fr[i]) <= tol or np.abs(fr[i]).max() == 0, "sequence %d final" % i


@pytest.mark.parametrize("name,over,chunk,lengths,label", CASES, ids=[c[4] for c in CASES])
def test_varlen_matches_oracle(name, over, chunk, lengths, label):
    _run(name, over, chunk, lengths, label)


def test_varlen_equals_batched_forward_for_equal_lengths():
    """Equal lengths: a packed batch is a [batch][seqlen] batch laid out flat; ssd_forward_varlen
    and ssd_forward take the same kernels and give the same bits."""
    cfg = ssd_inputs.config("mamba2_layer", batch=3, seqlen=300, nheads=4, init=True)
    announce("varlen equal lengths vs batched")
    inp = ssd_inputs.make_inputs(cfg, 43)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    yb, fb = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), chunk=128,
                             init_state=g["init_state"], final_state=True)
    cu = torch.arange(0, 4 * 300, 300, dtype=torch.int64, device="cuda")
    yv, fv, _ = ssd.ssd_forward_varlen(g["x"].reshape(900, 4, 64), g["log_a"].reshape(900, 4),
                                       g["B"].reshape(900, 1, 128), g["C"].reshape(900, 1, 128), cu, 300, g.get("D"),
                                       chunk=128, init_state=g["init_state"], final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(yv.reshape(3, 300, 4, 64), yb) and torch.equal(fv, fb)


def test_varlen_all_empty_and_clamped_offsets():
    """No tokens at all: every final state is its initial state.  Offsets past the token count and
    a sequence longer than max_seqlen are clamped (the header's contract): the result is that of the
    clamped sequences, and rows past the clamped end are left as they were."""
    cfg = ssd_inputs.config("mamba2_layer", nheads=2, init=True)
    announce("varlen all-empty")
    p = ssd_inputs.packed_inputs(cfg, [0, 0, 0], 44)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    _, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"], 0, g.get("D"),
                                       chunk=128, init_state=g["init_state"], final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(fin, g["init_state"])

    announce("varlen clamped offsets")
    p = ssd_inputs.packed_inputs(cfg, [50, 150], 45)      # 200 tokens
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    cu = torch.tensor([0, 50, 500], dtype=torch.int64, device="cuda")   # ends past the 200 tokens
    y = torch.full((200, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    _, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], cu, 120, g.get("D"), chunk=128,
                                       init_state=g["init_state"], y=y, final_state=True)
    torch.cuda.synchronize()
    # as the clamped batch: [0, 50) and [50, 170)
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"][:170]), f64(p["log_a"][:170]),
                                          f64(p["B"][:170]), f64(p["C"][:170]), np.array([0, 50, 170]),
                                          f64(p.get("D")), f64(p["init_state"]))
    assert rel_l2(y[:170].double().cpu().numpy(), yr) <= TOL["bf16"]
    assert rel_l2(fin.double().cpu().numpy(), fr) <= TOL["bf16"]
    assert bool((y[170:] == 7.0).all())


DT_CASES = [
    ("mamba2_layer", dict(nheads=4, init=True), 128, [300, 0, 129, 1000, 57], True, "fast-dt"),
    ("mamba2_layer", dict(nheads=4, init=False), 64, [70, 1, 640], False, "fast-dt-unscaled"),
    ("diag_multiscale", dict(nheads=2, init=True, a_log="rand_hn"), 64, [200, 0, 517], True, "diag-pipe-dt"),
    ("tiny_fp32", dict(nheads=3, skip=True, init=True, a_log="uniform16", dt_mean=-1.0), 64, [90, 0, 257, 1], True,
     "generic-fp32-dt"),
    ("diag_multiscale", dict(nheads=2, dstate=16, headdim=32, dtype="fp32", init=True, a_log="rand_hn"), 32,
     [77, 140], True, "generic-diag-fp32-dt"),
]


@pytest.mark.parametrize("name,over,chunk,lengths,scale,label", DT_CASES, ids=[c[5] for c in DT_CASES])
def test_dt_varlen_matches_oracle(name, over, chunk, lengths, scale, label):
    """ssd_forward_dt_varlen against the oracle's discretisation (oracle.discretize) followed by
    its per-sequence recurrence, with D x on the raw x."""
    cfg = ssd_inputs.config(name, **over)
    announce("dt varlen %s lengths=%s chunk=%d scale=%d" % (label, lengths, chunk, scale))
    p = ssd_inputs.packed_inputs(cfg, lengths, 47)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 48)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    y, fin, _ = ssd.ssd_forward_dt_varlen(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g["cu_seqlens"],
                                          p["max_seqlen"], g.get("D"), dt_bias=bias.cuda(), scale_input=scale,
                                          chunk=chunk, init_state=g.get("init_state"), final_state=True)
    torch.cuda.synchronize()
    diag = cfg["decay"] == "diag"
    delta, la = oracle.discretize.discretize(f64(p["dt"])[None], f64(p["A_log"]), f64(bias), diag)
    x = f64(p["x"])
    xin = x * delta[0][..., None] if scale else x
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), xin, la[0], f64(p["B"]), f64(p["C"]),
                                          p["cu_seqlens"].numpy(), None, f64(p.get("init_state")))
    if p.get("D") is not None:
        yr = yr + f64(p["D"])[None, :, None] * x
    tol = TOL[cfg["dtype"]]
    ey = rel_l2(y.double().cpu().numpy(), yr)
    ef = rel_l2(fin.double().cpu().numpy(), fr)
    announce("dt varlen %s: y %.2e final %.2e (tol %.0e)" % (label, ey, ef, tol))
    assert ey <= tol and ef <= tol, (ey, ef)


BWD_CASES = [
    ("mamba2_layer", dict(nheads=4, init=True), [300, 0, 129, 1000, 1, 57], "bwd-bf16-n128"),
    ("tiny_fp32", dict(nheads=3, skip=True, init=True, a_log="uniform16", dt_mean=-2.0), [90, 0, 257, 64], "bwd-fp32"),
    ("gqa_decode", dict(nheads=8, ngroups=2, init=True, decode_steps=0, dstate=64), [64, 700, 3], "bwd-bf16-gqa"),
    ("diag_multiscale", dict(nheads=3, init=True, a_log="rand_hn"), [200, 0, 64, 1, 517], "bwd-diag-bf16"),
    ("diag_multiscale", dict(nheads=2, ngroups=2, dstate=16, headdim=16, dtype="fp32", init=True, a_log="rand_hn"),
     [77, 0, 140], "bwd-diag-fp32"),
]


@pytest.mark.parametrize("name,over,lengths,label", BWD_CASES, ids=[c[3] for c in BWD_CASES])
def test_backward_varlen_matches_oracle(name, over, lengths, label):
    """ssd_backward_varlen against the oracle's per-sequence adjoint (oracle.varlen.backward_varlen):
    every gradient, with initial states and a gradient for every final state."""
    cfg = ssd_inputs.config(name, **over)
    announce("backward varlen %s lengths=%s" % (label, lengths))
    p = ssd_inputs.packed_inputs(cfg, lengths, 51)
    gen = torch.Generator().manual_seed(52)
    dy = torch.randn(p["x"].shape, generator=gen).to(p["x"].dtype)
    dfin = torch.randn((len(lengths), cfg["nheads"], cfg["dstate"], cfg["headdim"]), generator=gen)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    got = ssd.ssd_backward_varlen(g["x"], g["log_a"], g["B"], g["C"], dy.cuda(), g["cu_seqlens"], p["max_seqlen"],
                                  g.get("D"), init_state=g.get("init_state"), dfinal=dfin.cuda())
    torch.cuda.synchronize()
    want = oracle.varlen.backward_varlen(oracle.backward.default_adjoint(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                         f64(p["C"]), p["cu_seqlens"].numpy(), f64(p.get("D")),
                                         f64(p.get("init_state")), f64(dy), f64(dfin))
    tol = TOL[cfg["dtype"]]
    keys = ("dx", "dlog_a", "dB", "dC", "dinit") + (("dD",) if cfg["skip"] else ())
    errs = {k: rel_l2(got[k].double().cpu().numpy(), want[k]) for k in keys}
    announce("backward varlen %s: " % label + " ".join("%s %.2e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    assert all(e <= tol for e in errs.values()), errs


def test_backward_varlen_equals_batched_for_equal_lengths():
    """Equal lengths: the packed backward takes the same kernels as the batched one; every gradient
    but dB and dC (added atomically over heads, so their last bits may differ) comes out the same."""
    cfg = ssd_inputs.config("mamba2_layer", batch=3, seqlen=300, nheads=4, init=True)
    announce("backward varlen equal lengths vs batched")
    inp = ssd_inputs.make_inputs(cfg, 53)
    og = ssd_inputs.output_gradients(cfg, 54)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in dict(inp, **og).items()}
    gb = ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], g.get("D"), init_state=g["init_state"],
                          dfinal=g["dfinal"])
    cu = torch.arange(0, 4 * 300, 300, dtype=torch.int64, device="cuda")
    gv = ssd.ssd_backward_varlen(g["x"].reshape(900, 4, 64), g["log_a"].reshape(900, 4), g["B"].reshape(900, 1, 128),
                                 g["C"].reshape(900, 1, 128), g["dy"].reshape(900, 4, 64), cu, 300, g.get("D"),
                                 init_state=g["init_state"], dfinal=g["dfinal"])
    torch.cuda.synchronize()
    assert torch.equal(gv["dx"].reshape(gb["dx"].shape), gb["dx"])
    assert torch.equal(gv["dlog_a"].reshape(gb["dlog_a"].shape), gb["dlog_a"])
    assert torch.equal(gv["dinit"], gb["dinit"]) and torch.equal(gv["dD"], gb["dD"])
    for k in ("dB", "dC"):
        assert rel_l2(gv[k].reshape(gb[k].shape).double().cpu().numpy(), gb[k].double().cpu().numpy()) <= 1e-6


DT_BWD_CASES = [
    ("mamba2_layer", dict(nheads=4, init=True), [300, 0, 129, 57], True, "bwd-dt-bf16"),
    ("tiny_fp32", dict(nheads=3, skip=True, init=True, a_log="uniform16", dt_mean=-1.0), [90, 0, 257], False,
     "bwd-dt-fp32-unscaled"),
    ("diag_multiscale", dict(nheads=2, init=True, a_log="rand_hn"), [200, 1, 317], True, "bwd-dt-diag-bf16"),
]


@pytest.mark.parametrize("name,over,lengths,scale,label", DT_BWD_CASES, ids=[c[4] for c in DT_BWD_CASES])
def test_backward_dt_varlen_matches_oracle(name, over, lengths, scale, label):
    """ssd_backward_dt_varlen against the oracle's chain rule (oracle.discretize.backward_dt) run
    on every sequence by itself, the per-head sums (dA_log, d bias, dD) added over the sequences;
    the sums over tokens measured against the size of their terms, as in the batched test."""
    cfg = ssd_inputs.config(name, **over)
    diag = cfg["decay"] == "diag"
    announce("backward dt varlen %s lengths=%s scale=%d" % (label, lengths, scale))
    p = ssd_inputs.packed_inputs(cfg, lengths, 55)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 56)
    gen = torch.Generator().manual_seed(57)
    dy = torch.randn(p["x"].shape, generator=gen).to(p["x"].dtype)
    dfin = torch.randn((len(lengths), cfg["nheads"], cfg["dstate"], cfg["headdim"]), generator=gen)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    got = ssd.ssd_backward_dt_varlen(g["x"], g["dt"], g["A_log"], g["B"], g["C"], dy.cuda(), g["cu_seqlens"],
                                     p["max_seqlen"], g.get("D"), dt_bias=bias.cuda(), scale_input=scale,
                                     init_state=g.get("init_state"), dfinal=dfin.cuda())
    torch.cuda.synchronize()
    T, H = p["dt"].shape
    want = dict(dx=np.zeros(p["x"].shape), ddt=np.zeros((T, H)), dB=np.zeros(p["B"].shape), dC=np.zeros(p["C"].shape),
                dinit=np.zeros(dfin.shape), dA_log=np.zeros(p["A_log"].shape), ddt_bias=np.zeros(H), dD=np.zeros(H))
    mag = dict(dA_log=np.zeros(p["A_log"].shape), ddt_bias=np.zeros(H))
    adj = oracle.backward.default_adjoint()
    cu = p["cu_seqlens"].numpy()
    for i in range(len(lengths)):
        s, e = int(cu[i]), int(cu[i + 1])
        if e == s:
            want["dinit"][i] = f64(dfin[i])
            continue
        sl = lambda t: f64(t[s:e])[None]
        init = None if p.get("init_state") is None else f64(p["init_state"][i:i + 1])
        w = oracle.discretize.backward_dt(adj, sl(p["x"]), sl(p["dt"]), f64(p["A_log"]), sl(p["B"]), sl(p["C"]),
                                          f64(p.get("D")), dt_bias=f64(bias), scale_input=scale, init_state=init,
                                          dy=sl(dy), dfinal=f64(dfin[i:i + 1]), diag=diag)
        for k in ("dx", "ddt", "dB", "dC"):
            want[k][s:e] = w[k][0]
        want["dinit"][i] = w["dinit"][0]
        for k in ("dA_log", "ddt_bias", "dD"):
            want[k] += w[k]
        mag["ddt_bias"] += np.abs(w["ddt"][0]).sum(axis=0)
        delta, la = oracle.discretize.discretize(sl(p["dt"]), f64(p["A_log"]), f64(bias), diag)
        xin = sl(p["x"]) * delta[..., None] if scale else sl(p["x"])
        a = adj.backward(xin, la, sl(p["B"]), sl(p["C"]), None, init, sl(dy), f64(dfin[i:i + 1]))
        mag["dA_log"] += np.abs(a["dlog_a"] * la).sum(axis=(0, 1))
    tol = TOL[cfg["dtype"]]
    errs = {k: rel_l2(got[k].double().cpu().numpy(), want[k]) for k in ("dx", "ddt", "dB", "dC", "dinit", "dD")}
    for k in ("dA_log", "ddt_bias"):
        errs[k] = float(np.linalg.norm(got[k].double().cpu().numpy() - want[k]) / np.linalg.norm(mag[k]))
    announce("backward dt varlen %s: " % label + " ".join("%s %.2e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    assert all(e <= tol for e in errs.values()), errs


@pytest.mark.parametrize("name,over,chunk,label", [
    ("diag_multiscale", dict(nheads=2, init=True), 64, "diag-pipe"),
    ("tiny_fp32", dict(nheads=2, skip=True, init=True), 64, "generic-fp32"),
    ("diag_multiscale", dict(nheads=2, dstate=16, headdim=32, dtype="fp32", init=True), 32, "generic-diag-fp32"),
], ids=["diag-pipe", "generic-fp32", "generic-diag-fp32"])
def test_varlen_clamped_offsets_other_paths(name, over, chunk, label):
    """The clamping contract on the diagonal and generic paths: offsets past the token count and a
    sequence longer than max_seqlen give the clamped sequences' results, rows past the clamped end
    untouched."""
    cfg = ssd_inputs.config(name, **over)
    announce("varlen clamped offsets %s" % label)
    p = ssd_inputs.packed_inputs(cfg, [50, 150], 58)      # 200 tokens
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    cu = torch.tensor([0, 50, 500], dtype=torch.int64, device="cuda")
    y = torch.full(p["x"].shape, 7.0, dtype=p["x"].dtype, device="cuda")
    _, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], cu, 120, g.get("D"), chunk=chunk,
                                       init_state=g["init_state"], y=y, final_state=True)
    torch.cuda.synchronize()
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"][:170]), f64(p["log_a"][:170]),
                                          f64(p["B"][:170]), f64(p["C"][:170]), np.array([0, 50, 170]),
                                          f64(p.get("D")), f64(p["init_state"]))
    tol = TOL[cfg["dtype"]]
    assert rel_l2(y[:170].double().cpu().numpy(), yr) <= tol
    assert rel_l2(fin.double().cpu().numpy(), fr) <= tol
    assert bool((y[170:] == 7.0).all())


def test_varlen_one_long_sequence():
    """One 65 536-token sequence among short ones: a packed batch is never segmented, so one
    workgroup per head walks all 512 of its chunks (the batched walk would split it)."""
    cfg = ssd_inputs.config("long_seq", nheads=2, init=True)
    lengths = [65536, 3, 700]
    announce("varlen one long sequence %s" % lengths)
    p = ssd_inputs.packed_inputs(cfg, lengths, 59)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    y, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"], p["max_seqlen"],
                                       g.get("D"), chunk=256, init_state=g["init_state"], final_state=True)
    torch.cuda.synchronize()
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                          f64(p["C"]), p["cu_seqlens"].numpy(), f64(p.get("D")), f64(p["init_state"]))
    ey, ef = rel_l2(y.double().cpu().numpy(), yr), rel_l2(fin.double().cpu().numpy(), fr)
    announce("varlen one long sequence: y %.2e final %.2e" % (ey, ef))
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("name,over,chunk", [("mamba2_layer", dict(nheads=4, init=True), 128),
                                             ("diag_multiscale", dict(nheads=2, init=True), 64)],
                         ids=["fast", "diag-pipe"])
def test_varlen_packing_order_is_irrelevant(name, over, chunk):
    """The same sequences packed in another order (so ranked and scheduled differently) give the
    same outputs and final states bit for bit: every (sequence, head) is computed by itself."""
    cfg = ssd_inputs.config(name, **over)
    lengths = [300, 17, 0, 1000, 129, 64, 5]
    announce("varlen packing order %s" % name)
    p = ssd_inputs.packed_inputs(cfg, lengths, 61)
    perm = [3, 0, 6, 2, 5, 1, 4]
    cu = p["cu_seqlens"]
    cat = lambda t: torch.cat([t[int(cu[i]):int(cu[i + 1])] for i in perm])
    q = {k: cat(p[k]) for k in ("x", "log_a", "B", "C")}
    cu2 = torch.zeros(len(perm) + 1, dtype=torch.int64)
    cu2[1:] = torch.cumsum(torch.tensor([lengths[i] for i in perm]), 0)
    init = p["init_state"]
    run = lambda d, c, h0: ssd.ssd_forward_varlen(d["x"].cuda(), d["log_a"].cuda(), d["B"].cuda(), d["C"].cuda(),
                                                 c.cuda(), max(lengths), p["D"].cuda(), chunk=chunk,
                                                 init_state=h0.cuda(), final_state=True)
    y1, f1, _ = run(p, cu, init)
    y2, f2, _ = run(q, cu2, init[perm])
    torch.cuda.synchronize()
    assert torch.equal(cat(y1.cpu()), y2.cpu())
    assert torch.equal(f1.cpu()[perm], f2.cpu())
