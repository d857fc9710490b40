"""Every path with its workspace filled with NaN bit patterns (all bytes 0xFF: a NaN as fp32
and as bf16) before the call, against the oracle.  A kernel that reads a workspace record
nobody wrote (a prep record past a short chunk, a segment state, a padded chunk's decay, a
backward checkpoint) would carry the NaN into its outputs.  Ragged lengths throughout."""
import numpy as np
import pytest
import torch

import oracle
import oracle.backward
import oracle.discretize
import oracle.varlen
import ssd_chunked_scan_02_amd as ssd
import ssd_inputs
from gpu_helpers import announce, compare, oracle_forward, rel_l2, to_gpu, TOL

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64


def _poisoned(nbytes):
    return torch.full((max(1, nbytes),), 0xFF, dtype=torch.uint8, device="cuda")


FORWARD = [
    ("mamba2_layer", dict(batch=2, seqlen=333, nheads=4, init=True), "fast"),
    ("mamba2_layer", dict(batch=2, seqlen=301, nheads=4, ngroups=2, dstate=64, chunk=64), "fast-n64"),
    ("mamba2_layer", dict(batch=1, seqlen=3001, nheads=2, init=True), "fast-segmented"),
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=3, init=True), "diag-pipe"),
    ("diag_multiscale", dict(batch=1, seqlen=2001, nheads=2, init=True), "diag-pipe-segmented"),
    ("tiny_fp32", dict(seqlen=250, skip=True, init=True), "generic-fp32"),
    ("diag_multiscale", dict(batch=1, seqlen=190, nheads=2, dtype="fp32", dstate=32, headdim=32, chunk=32,
                             init=True), "generic-diag"),
]


@pytest.mark.parametrize("name,over,label", FORWARD, ids=[c[2] for c in FORWARD])
def test_forward_with_poisoned_workspace(name, over, label):
    cfg = ssd_inputs.config(name, **over)
    announce("poisoned workspace: forward %s" % label)
    inp = ssd_inputs.make_inputs(cfg, 101)
    g = to_gpu(inp)
    dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
    ws = _poisoned(ssd.ssd_forward_workspace_bytes(dims, cfg["chunk"]))
    for rep in range(2):  # the second call finds the first call's records in place
        y, fin = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), chunk=cfg["chunk"],
                                 init_state=g.get("init_state"), final_state=True, workspace=ws)
        torch.cuda.synchronize()
        compare(inp, y, fin, oracle_forward(inp), cfg["dtype"], True, "poisoned %s #%d" % (label, rep))
        ws.fill_(0xFF)


DT = [
    ("mamba2_layer", dict(batch=2, seqlen=333, nheads=4, init=True), "fast"),
    ("mamba2_layer", dict(batch=1, seqlen=3001, nheads=2, init=True), "fast-segmented"),
    ("diag_multiscale", dict(batch=2, seqlen=300, nheads=3, a_log="rand_hn", init=True), "diag-pipe"),
    ("tiny_fp32", dict(seqlen=250, skip=True, init=True, nheads=2, a_log="uniform16"), "generic-fp32"),
]


@pytest.mark.parametrize("name,over,label", DT, ids=[c[2] for c in DT])
def test_forward_dt_with_poisoned_workspace(name, over, label):
    cfg = ssd_inputs.config(name, **over)
    diag = cfg["decay"] == "diag"
    announce("poisoned workspace: forward_dt %s" % label)
    inp = ssd_inputs.make_inputs(cfg, 103)
    bias = ssd_inputs.dt_bias(cfg["nheads"], 203)
    g = to_gpu(inp)
    dims = ssd.Dims(*g["x"].shape[:3], g["B"].shape[2], g["x"].shape[3], g["B"].shape[3],
                    ssd.SSD_BF16 if cfg["dtype"] == "bf16" else ssd.SSD_F32,
                    ssd.SSD_DECAY_DIAG if diag else ssd.SSD_DECAY_SCALAR)
    ws = _poisoned(ssd.ssd_forward_dt_workspace_bytes(dims, cfg["chunk"], True))
    y, fin = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"), dt_bias=bias.cuda(),
                                scale_input=True, chunk=cfg["chunk"], init_state=g.get("init_state"),
                                final_state=True, workspace=ws)
    torch.cuda.synchronize()
    yr, fr = oracle.discretize.forward_dt(oracle.default_oracle(), f64(inp["x"]), f64(inp["dt"]), f64(inp["A_log"]),
                                          f64(inp["B"]), f64(inp["C"]), f64(inp.get("D")), dt_bias=f64(bias),
                                          scale_input=True, init_state=f64(inp.get("init_state")), diag=diag)
    ref = {(b, h): (yr[b, :, h], fr[b, h]) for b in range(yr.shape[0]) for h in range(yr.shape[2])}
    compare(inp, y, fin, ref, cfg["dtype"], True, "poisoned dt %s" % label)


VARLEN = [
    ("mamba2_layer", dict(nheads=4, init=True), 128, [300, 1, 0, 129, 77], "fast"),
    ("diag_multiscale", dict(nheads=3, init=True), 64, [200, 0, 65, 1], "diag-pipe"),
    ("tiny_fp32", dict(nheads=3, skip=True, init=True), 64, [90, 0, 257], "generic-fp32"),
]


@pytest.mark.parametrize("name,over,chunk,lengths,label", VARLEN, ids=[c[4] for c in VARLEN])
def test_varlen_with_poisoned_workspace(name, over, chunk, lengths, label):
    cfg = ssd_inputs.config(name, **over)
    announce("poisoned workspace: varlen %s lengths=%s" % (label, lengths))
    p = ssd_inputs.packed_inputs(cfg, lengths, 107)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    dims = ssd.varlen_dims(g["x"], g["log_a"], g["B"], len(lengths), p["max_seqlen"])
    ws = _poisoned(ssd.ssd_forward_varlen_workspace_bytes(dims, chunk))
    y, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"], p["max_seqlen"],
                                       g.get("D"), chunk=chunk, init_state=g.get("init_state"), final_state=True,
                                       workspace=ws)
    torch.cuda.synchronize()
    yr, fr = oracle.varlen.forward_varlen(oracle.default_oracle(), f64(p["x"]), f64(p["log_a"]), f64(p["B"]),
                                          f64(p["C"]), p["cu_seqlens"].numpy(), f64(p.get("D")),
                                          f64(p.get("init_state")))
    tol = TOL[cfg["dtype"]]
    ey, ef = rel_l2(y.double().cpu().numpy(), yr), rel_l2(fin.double().cpu().numpy(), fr)
    announce("poisoned varlen %s: y %.2e final %.2e (tol %.0e)" % (label, ey, ef, tol))
    assert np.isfinite(ey) and np.isfinite(ef) and ey <= tol and ef <= tol


BACKWARD = [
    ("mamba2_layer", dict(batch=2, seqlen=301, nheads=4, init=True), "scalar-bf16"),
    ("tiny_fp32", dict(seqlen=201, init=True, skip=True), "scalar-fp32"),
    ("diag_multiscale", dict(batch=2, seqlen=301, nheads=3, a_log="rand_hn", init=True), "diag-bf16"),
]


@pytest.mark.parametrize("name,over,label", BACKWARD, ids=[c[2] for c in BACKWARD])
def test_backward_with_poisoned_workspace(name, over, label):
    cfg = ssd_inputs.config(name, **over)
    announce("poisoned workspace: backward %s" % label)
    inp = ssd_inputs.make_inputs(cfg, 109)
    og = ssd_inputs.output_gradients(cfg, 209)
    g = to_gpu(dict(inp, **og))
    dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
    ws = _poisoned(ssd.ssd_backward_workspace_bytes(dims))
    got = ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], g.get("D"), init_state=g.get("init_state"),
                           dfinal=g["dfinal"], workspace=ws)
    torch.cuda.synchronize()
    want = oracle.backward.backward(f64(inp["x"]), f64(inp["log_a"]), f64(inp["B"]), f64(inp["C"]),
                                    f64(inp.get("D")), f64(inp.get("init_state")), f64(og["dy"]), f64(og["dfinal"]))
    tol = TOL[cfg["dtype"]]
    keys = ("dx", "dlog_a", "dB", "dC", "dinit") + (("dD",) if cfg["skip"] else ())
    errs = {k: rel_l2(got[k].double().cpu().numpy(), want[k]) for k in keys}
    announce("poisoned backward %s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    for k, e in errs.items():
        assert np.isfinite(e) and e <= tol, (k, e)
