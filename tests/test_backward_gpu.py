"""ssd_backward on the GPU against the fp64 adjoint (oracle/backward.py), gradient by gradient,
on the same seeded inputs and output gradients.  Bounds as for the forward pass: relative L2
<= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs, on dx, dlog a, dB, dC, dD and dinit."""
import numpy as np
import pytest
import torch

import oracle.backward
import oracle.discretize
import ssd_chunked_scan_02_amd as ssd
import ssd_inputs
from gpu_helpers import announce, rel_l2, to_gpu, TOL

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64

CASES = [
    ("tiny_fp32", dict(seqlen=200, init=True, skip=True), "fp32-n16"),
    ("tiny_fp32", dict(seqlen=100, nheads=4, ngroups=2, dstate=64, headdim=32, init=True, skip=True,
                       a_log="uniform16"), "fp32-groups"),
    ("mamba2_layer", dict(batch=2, seqlen=300, nheads=4), "bf16-n128"),
    ("mamba2_layer", dict(batch=2, seqlen=150, nheads=4, ngroups=2, dstate=64, init=True), "bf16-n64-init"),
    ("mamba2_layer", dict(batch=1, seqlen=77, nheads=2, dstate=32, headdim=16, init=True, dt_mean=-8.0), "bf16-slow"),
    ("mamba2_layer", dict(batch=1, seqlen=64, nheads=2, dt_mean=3.0), "bf16-fast"),
    # many backward chunks and a ragged tail; eight heads per group (dB, dC summed over them)
    ("gqa_decode", dict(batch=2, seqlen=1500, nheads=16, ngroups=2, decode_steps=0, init=True), "bf16-long-gqa"),
    # the other shapes of the bf16-MFMA backward kernels (N in {32, 64, 128}, P in {32, 64})
    ("mamba2_layer", dict(batch=2, seqlen=200, nheads=4, ngroups=2, dstate=32, headdim=32, init=True), "bf16-n32-p32"),
    ("mamba2_layer", dict(batch=1, seqlen=160, nheads=3, dstate=32, headdim=64, init=True), "bf16-n32-p64"),
    ("mamba2_layer", dict(batch=1, seqlen=160, nheads=2, dstate=64, headdim=32), "bf16-n64-p32"),
    ("mamba2_layer", dict(batch=2, seqlen=97, nheads=2, dstate=128, headdim=32, init=True), "bf16-n128-p32"),
    ("tiny_fp32", dict(batch=2, seqlen=1100, nheads=2, dstate=128, headdim=64, init=True, skip=True,
                       a_log="uniform16", dt_mean=-2.0), "fp32-long"),
    # diagonal decay: per-(head, dim) rates, fast and slow dimensions in one head
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=3, a_log="rand_hn", init=True), "diag-bf16"),
    ("diag_multiscale", dict(batch=1, seqlen=500, nheads=2, dstate=32, headdim=32, init=True), "diag-bf16-32"),
    ("diag_multiscale", dict(batch=2, seqlen=170, nheads=2, ngroups=2, dstate=16, headdim=16, dtype="fp32",
                             a_log="rand_hn", init=True), "diag-fp32"),
    ("diag_multiscale", dict(batch=1, seqlen=130, nheads=2, dtype="fp32", init=True), "diag-fp32-64"),
    # extreme rates: whole blocks decay to exact zeros (fast), or nothing decays (slow)
    ("diag_multiscale", dict(batch=1, seqlen=200, nheads=2, a_log="rand_hn", dt_mean=3.0, init=True), "diag-fast"),
    ("diag_multiscale", dict(batch=1, seqlen=200, nheads=2, dt_mean=-8.0, init=True), "diag-slow"),
    # lopsided shapes: one 16-wide block of state dims, or of head dims
    ("diag_multiscale", dict(batch=2, seqlen=150, nheads=2, dstate=64, headdim=16, init=True), "diag-n64-p16"),
    ("diag_multiscale", dict(batch=2, seqlen=150, nheads=2, dstate=16, headdim=64, init=True), "diag-n16-p64"),
]


@pytest.mark.parametrize("name,over,label", CASES, ids=[c[2] for c in CASES])
def test_backward_matches_adjoint(name, over, label):
    cfg = ssd_inputs.config(name, **over)
    announce("backward %s cfg=%s" % (label, {k: cfg[k] for k in ("batch", "seqlen", "nheads", "ngroups", "headdim",
                                                                   "dstate", "dtype", "init", "skip")}))
    inp = ssd_inputs.make_inputs(cfg, 71)
    og = ssd_inputs.output_gradients(cfg, 171)
    g = to_gpu(dict(inp, **og))
    got = ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], g.get("D"), init_state=g.get("init_state"),
                           dfinal=g["dfinal"])
    torch.cuda.synchronize()
    want = oracle.backward.backward(f64(inp["x"]), f64(inp["log_a"]), f64(inp["B"]), f64(inp["C"]), f64(inp.get("D")),
                                    f64(inp.get("init_state")), f64(og["dy"]), f64(og["dfinal"]))
    tol = TOL[cfg["dtype"]]
    errs = {}
    for k in ("dx", "dlog_a", "dB", "dC", "dinit") + (("dD",) if cfg["skip"] else ()):
        errs[k] = rel_l2(got[k].double().cpu().numpy(), want[k])
    announce("backward %s: " % label + " ".join("%s %.2e" % kv for kv in errs.items()) + " (tol %.0e)" % tol)
    assert all(np.isfinite(got[k].float().cpu().numpy()).all() for k in errs)
    assert all(e <= tol for e in errs.values()), errs


def test_backward_optional_arguments():
    """No D, no initial state, no dfinal; dD and dinit not requested: the gradients of
    <dy, y> alone (the oracle with zeros in their place)."""
    cfg = ssd_inputs.config("mamba2_layer", batch=1, seqlen=130, nheads=2, skip=False)
    announce("backward optional arguments")
    inp = ssd_inputs.make_inputs(cfg, 73)
    og = ssd_inputs.output_gradients(cfg, 173)
    g = to_gpu(dict(inp, **og))
    got = ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], want_dD=False, want_dinit=False)
    torch.cuda.synchronize()
    want = oracle.backward.backward(f64(inp["x"]), f64(inp["log_a"]), f64(inp["B"]), f64(inp["C"]), None, None,
                                    f64(og["dy"]), None)
    assert got["dD"] is None and got["dinit"] is None
    for k in ("dx", "dlog_a", "dB", "dC"):
        e = rel_l2(got[k].double().cpu().numpy(), want[k])
        assert e <= TOL["bf16"], (k, e)


def test_backward_empty_sequence():
    """T = 0: dinit = dfinal, dD = 0, nothing else to write."""
    cfg = ssd_inputs.config("tiny_fp32", seqlen=0, init=True, skip=True)
    announce("backward empty sequence")
    x = torch.zeros((1, 0, 1, 64), device="cuda")
    la = torch.zeros((1, 0, 1), device="cuda")
    Bm = torch.zeros((1, 0, 1, 16), device="cuda")
    dfinal = torch.randn((1, 1, 16, 64), device="cuda")
    got = ssd.ssd_backward(x, la, Bm, Bm.clone(), x.clone(), torch.ones(1, device="cuda"),
                           init_state=torch.ones((1, 1, 16, 64), device="cuda"), dfinal=dfinal)
    torch.cuda.synchronize()
    assert torch.equal(got["dinit"], dfinal) and float(got["dD"][0]) == 0.0


DT_CASES = [
    ("mamba2_layer", dict(batch=2, seqlen=300, nheads=4, init=True), "bf16"),
    ("gqa_decode", dict(batch=1, seqlen=700, nheads=8, ngroups=2, decode_steps=0, init=True), "bf16-gqa"),
    ("tiny_fp32", dict(seqlen=200, nheads=2, skip=True, init=True, a_log="uniform16", dt_mean=-1.0), "fp32"),
    # diagonal decay: A_log [H,N]
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=3, a_log="rand_hn", init=True), "diag-bf16"),
    ("diag_multiscale", dict(batch=1, seqlen=170, nheads=2, dstate=32, headdim=16, dtype="fp32", a_log="rand_hn",
                             init=True), "diag-fp32"),
]


@pytest.mark.parametrize("scale", [True, False], ids=["scaled", "unscaled"])
@pytest.mark.parametrize("name,over,label", DT_CASES, ids=[c[2] for c in DT_CASES])
def test_backward_dt_matches_chain_rule(name, over, label, scale):
    """ssd_backward_dt against the oracle's chain rule through the discretisation
    (oracle.discretize.backward_dt on the fp64 adjoint), every gradient."""
    cfg = ssd_inputs.config(name, **over)
    announce("backward_dt %s scale=%d" % (label, scale))
    inp = ssd_inputs.make_inputs(cfg, 75)
    og = ssd_inputs.output_gradients(cfg, 175)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 275)
    g = to_gpu(dict(inp, **og))
    got = ssd.ssd_backward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g["dy"], g.get("D"), dt_bias=bias.cuda(),
                              scale_input=scale, init_state=g.get("init_state"), dfinal=g["dfinal"])
    torch.cuda.synchronize()
    diag = cfg["decay"] == "diag"
    want = oracle.discretize.backward_dt(oracle.backward.default_adjoint(), f64(inp["x"]), f64(inp["dt"]),
                                         f64(inp["A_log"]), f64(inp["B"]), f64(inp["C"]), f64(inp.get("D")),
                                         dt_bias=f64(bias), scale_input=scale, init_state=f64(inp.get("init_state")),
                                         dy=f64(og["dy"]), dfinal=f64(og["dfinal"]), diag=diag)
    tol = TOL[cfg["dtype"]]
    errs = {k: rel_l2(got[k].double().cpu().numpy(), want[k]) for k in ("dx", "ddt", "dB", "dC", "dD", "dinit")}
    # dA_log and ddt_bias are sums over every (batch, token) of terms of both signs: their error is
    # measured against the size of the terms (sum of magnitudes per head), since cancellation in
    # the sum can leave it far smaller than the rounding its terms carry
    la = oracle.discretize.discretize(f64(inp["dt"]), f64(inp["A_log"]), f64(bias), diag)[1]
    mag = dict(ddt_bias=np.abs(want["ddt"]).sum(axis=(0, 1)))
    # the dA_log terms are dlog_a log a: dlog_a from the adjoint on the same inputs
    xin = f64(inp["x"]) * oracle.discretize.discretize(f64(inp["dt"]), f64(inp["A_log"]), f64(bias), diag)[0][..., None] \
        if scale else f64(inp["x"])
    adj = oracle.backward.backward(xin, la, f64(inp["B"]), f64(inp["C"]), None, f64(inp.get("init_state")),
                                   f64(og["dy"]), f64(og["dfinal"]))
    mag["dA_log"] = np.abs(adj["dlog_a"] * la).sum(axis=(0, 1))
    for k in ("dA_log", "ddt_bias"):
        diff = got[k].double().cpu().numpy() - want[k]
        errs[k] = float(np.linalg.norm(diff) / np.linalg.norm(mag[k]))
    announce("backward_dt %s scale=%d: " % (label, scale) + " ".join("%s %.2e" % kv for kv in errs.items())
             + " (tol %.0e)" % tol)
    assert all(e <= tol for e in errs.values()), errs
