"""The discretisation front-end (ssd_forward_dt, ssd_step_dt) on the GPU against the fp64
oracle's front-end (oracle.discretize: Delta = softplus(dt + bias), log a = -Delta exp(A_log),
input term Delta B x^T, skip on the raw x), element by element on the same seeded inputs.

Covers the fused paths (the bf16 scalar fast path, plain and segmented; the pipelined diagonal
walk, plain and segmented), the generic composition (fp32 and other shapes: log a and the
scaled input written to the workspace, then the walk, then the skip term), with and without the
input scale and the bias, ragged tails, and decode steps continuing a forward pass.  Bounds as
for ssd_forward: relative L2 <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
import oracle.discretize
import ssd_chunked_scan_02_amd as ssd
import ssd_inputs
from gpu_helpers import announce, compare, rel_l2, to_gpu, TOL

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64


def _oracle_dt(inp, bias, scale, diag):
    y, fin = oracle.discretize.forward_dt(
        oracle.default_oracle(), f64(inp["x"]), f64(inp["dt"]), f64(inp["A_log"]), f64(inp["B"]),
        f64(inp["C"]), f64(inp.get("D")), dt_bias=f64(bias), scale_input=scale,
        init_state=f64(inp.get("init_state")), diag=diag)
    nb, H = y.shape[0], y.shape[2]
    return {(b, h): (y[b, :, h], fin[b, h]) for b in range(nb) for h in range(H)}


def _run(name, over, seed, scale, with_bias, label):
    cfg = ssd_inputs.config(name, **over)
    diag = cfg["decay"] == "diag"
    announce("%s seed=%d scale=%d bias=%d cfg=%s" % (label, seed, scale, with_bias, {
        k: cfg[k] for k in ("batch", "seqlen", "nheads", "ngroups", "headdim", "dstate", "chunk", "dtype",
                            "decay", "a_log", "dt_mean")}))
    inp = ssd_inputs.make_inputs(cfg, seed)
    bias = ssd_inputs.dt_bias(cfg["nheads"], seed + 100) if with_bias else None
    g = to_gpu(inp)
    y, fin = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"),
                                dt_bias=None if bias is None else bias.cuda(), scale_input=scale,
                                chunk=cfg["chunk"], init_state=g.get("init_state"), final_state=True)
    torch.cuda.synchronize()
    ref = _oracle_dt(inp, bias, scale, diag)
    return compare(inp, y, fin, ref, cfg["dtype"], True, label)


CASES = [
    # bf16 scalar fast path (N 128, chunk 128; N 64, chunk 64 with two groups), ragged tails
    ("mamba2_layer", dict(batch=2, seqlen=600, nheads=4, init=True), "fast"),
    ("mamba2_layer", dict(batch=2, seqlen=333, nheads=4, ngroups=2, dstate=64, chunk=64), "fast-n64"),
    ("mamba2_layer", dict(batch=1, seqlen=700, nheads=3, chunk=256, init=True), "fast-q256"),
    # ... segmented (few units, long sequence): slow and fast decay, so that the state pass runs
    # every chunk and stops early
    ("mamba2_layer", dict(batch=1, seqlen=3000, nheads=2, init=True), "fast-seg"),
    ("mamba2_layer", dict(batch=1, seqlen=3000, nheads=2, init=True, dt_mean=-8.0), "fast-seg-slow"),
    ("mamba2_layer", dict(batch=1, seqlen=3000, nheads=2, init=True, dt_mean=2.0), "fast-seg-fast"),
    # pipelined diagonal walk (bf16, chunk 64), per-(head, dim) rates, plain and segmented
    ("diag_multiscale", dict(batch=2, seqlen=600, nheads=3, a_log="rand_hn", init=True), "diag"),
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=2, headdim=32, dstate=32), "diag-32"),
    ("diag_multiscale", dict(batch=1, seqlen=2500, nheads=2, a_log="rand_hn", init=True), "diag-seg"),
    # generic composition: fp32 scalar, bf16 scalar outside the fast path, fp32 diagonal
    ("tiny_fp32", dict(seqlen=250, skip=True, init=True, nheads=2, a_log="uniform16"), "generic-fp32"),
    ("mamba2_layer", dict(batch=2, seqlen=300, nheads=4, headdim=32, dstate=64, chunk=64), "generic-bf16"),
    ("diag_multiscale", dict(batch=1, seqlen=200, nheads=2, headdim=32, dstate=16, chunk=32, dtype="fp32",
                             a_log="rand_hn", init=True), "generic-diag-fp32"),
]


@pytest.mark.parametrize("scale", [True, False], ids=["scaled", "unscaled"])
@pytest.mark.parametrize("name,over,label", CASES, ids=[c[2] for c in CASES])
def test_forward_dt(name, over, label, scale):
    _run(name, over, 41, scale, True, "dt " + label)


@pytest.mark.parametrize("label", ["fast", "diag", "generic-fp32"])
def test_forward_dt_without_bias(label):
    name, over, _ = next(c for c in CASES if c[2] == label)
    _run(name, over, 43, True, False, "dt no-bias " + label)


def test_forward_dt_matches_forward_on_its_log_a():
    """Without the input scale, ssd_forward_dt is ssd_forward on log a = -softplus(dt) exp(A_log):
    the two GPU results agree to the bf16 rounding of y (their log a differ only by fp32
    rounding of the front-end)."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=520, nheads=4)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 47))
    announce("dt vs log_a")
    y0, f0 = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g["D"], chunk=128, final_state=True)
    y1, f1 = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g["D"], scale_input=False,
                                chunk=128, final_state=True)
    torch.cuda.synchronize()
    e_y = rel_l2(y1.float().cpu().numpy(), y0.float().cpu().numpy())
    e_f = rel_l2(f1.cpu().numpy(), f0.cpu().numpy())
    announce("dt vs log_a: y %.2e final %.2e" % (e_y, e_f))
    assert e_y < 1e-3 and e_f < 1e-4


@pytest.mark.parametrize("name,over,launches", [
    ("mamba2_layer", dict(batch=2, seqlen=520, nheads=4), 2),                          # prep, walk
    ("mamba2_layer", dict(batch=1, seqlen=3000, nheads=2), 3),                         # + state pass
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=2), 1),                       # walk
    ("tiny_fp32", dict(skip=True), 4),                                                 # disc, scores, walk, skip
], ids=["fast", "fast-seg", "diag", "generic"])
def test_profiled_dt_launches(name, over, launches):
    """ssd_forward_dt_profiled stamps one event pair per launch and gives ssd_forward_dt's
    outputs bit for bit."""
    from bench import HipEvents
    cfg = ssd_inputs.config(name, **over)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 53))
    announce("profiled dt %s %s" % (name, over))
    kw = dict(chunk=cfg["chunk"], final_state=True)
    y0, f0 = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"), **kw)
    ev = HipEvents()
    events = [ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)]
    try:
        y1, f1, n = ssd.ssd_forward_dt_profiled(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"),
                                                events=events, **kw)
        torch.cuda.synchronize()
        assert n == launches
        times = [ev.elapsed_ms(events[2 * k], events[2 * k + 1]) for k in range(n)]
        assert all(0.0 < t < 1000.0 for t in times), times
    finally:
        for e in events:
            ev.destroy(e)
    assert torch.equal(y0.float(), y1.float()) and torch.equal(f0, f1)


@pytest.mark.parametrize("name,over", [
    ("gqa_decode", dict(batch=2, seqlen=300, nheads=8, ngroups=2, decode_steps=24)),
    ("diag_multiscale", dict(batch=2, seqlen=130, nheads=2, a_log="rand_hn", dtype="fp32", decode_steps=24)),
], ids=["scalar-bf16", "diag-fp32"])
def test_step_dt_continues_forward_dt(name, over):
    """forward_dt(T) then k steps of step_dt equals the oracle's front-end over T + k tokens,
    y of every step and the final state."""
    cfg = ssd_inputs.config(name, **over)
    diag = cfg["decay"] == "diag"
    inp = ssd_inputs.make_inputs(cfg, 59)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 159)
    g = to_gpu(inp)
    announce("step_dt %s %s" % (name, over))
    _, state = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"), dt_bias=bias.cuda(),
                                  chunk=cfg["chunk"], final_state=True)
    ys = []
    for t in range(cfg["decode_steps"]):
        ys.append(ssd.ssd_step_dt(state, g["x_dec"][:, t].contiguous(), g["dt_dec"][:, t].contiguous(), g["A_log"],
                                  g["B_dec"][:, t].contiguous(), g["C_dec"][:, t].contiguous(), g.get("D"),
                                  dt_bias=bias.cuda()).clone())
    torch.cuda.synchronize()
    whole = {k: torch.cat([inp[k], inp[k + "_dec"]], 1) for k in ("x", "dt", "B", "C")}
    y_ref, f_ref = oracle.discretize.forward_dt(
        oracle.default_oracle(), f64(whole["x"]), f64(whole["dt"]), f64(inp["A_log"]), f64(whole["B"]),
        f64(whole["C"]), f64(inp.get("D")), dt_bias=f64(bias), diag=diag)
    T = cfg["seqlen"]
    y_dec = np.stack([y.float().cpu().numpy() for y in ys], 1)
    e_y = rel_l2(y_dec, y_ref[:, T:])
    e_f = rel_l2(state.cpu().numpy(), f_ref)
    tol = TOL[cfg["dtype"]]
    announce("step_dt %s: y %.2e final %.2e (tol %.0e)" % (name, e_y, e_f, tol))
    assert e_y <= tol and e_f <= tol
