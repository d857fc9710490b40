"""Full-size checks of the backward pass, the packed batches and the discretisation front-end, in
the launch configuration bench.py times, on outputs the oracle computes in seconds: the backward
pass over the whole workload compared on batch element 0 (its dx, d log a, dB, dC and d init depend
on that element alone), the 32-sequence packed batch of ``bench.py --varlen 32`` compared on sampled
sequences (the shortest, the longest and two others), and the front-end's forward over the whole
workload, every output.  Bounds as everywhere: relative L2 <= 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
import oracle.backward
import ssd_chunked_scan_02_amd as ssd
import ssd_inputs
from gpu_helpers import announce, rel_l2, to_gpu, TOL

pytestmark = pytest.mark.gpu

f64 = ssd_inputs.to_f64


@pytest.mark.parametrize("name", ["mamba2_layer", "diag_multiscale"])
def test_backward_full_workload_batch0(name):
    cfg = ssd_inputs.config(name)
    announce("full backward %s (oracle on batch element 0)" % name)
    inp = ssd_inputs.make_inputs(cfg, ssd_inputs.SEEDS[name])
    og = ssd_inputs.output_gradients(cfg, ssd_inputs.SEEDS[name] + 1000)
    g = to_gpu(dict(inp, **og))
    got = ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], g.get("D"), init_state=g.get("init_state"),
                           dfinal=g["dfinal"] if cfg["final"] else None)
    torch.cuda.synchronize()
    one = lambda t: None if t is None else f64(t[:1])
    want = oracle.backward.backward(one(inp["x"]), one(inp["log_a"]), one(inp["B"]), one(inp["C"]), f64(inp.get("D")),
                                    one(inp.get("init_state")), one(og["dy"]),
                                    one(og["dfinal"]) if cfg["final"] else None)
    errs = {k: rel_l2(got[k][:1].double().cpu().numpy(), want[k]) for k in ("dx", "dlog_a", "dB", "dC", "dinit")}
    announce("full backward %s: " % name + " ".join("%s %.2e" % kv for kv in errs.items()))
    assert all(e <= TOL[cfg["dtype"]] for e in errs.values()), errs


def test_varlen_bench_batch_sampled():
    cfg = ssd_inputs.config("mamba2_layer")
    seed = ssd_inputs.SEEDS["mamba2_layer"]
    lengths = ssd_inputs.packed_lengths(32, cfg["batch"] * cfg["seqlen"], seed)
    announce("full varlen: 32 sequences, lengths %d..%d" % (min(lengths), max(lengths)))
    p = ssd_inputs.packed_inputs(cfg, lengths, seed)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    y, fin, _ = ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], g["cu_seqlens"], p["max_seqlen"],
                                       g.get("D"), chunk=cfg["chunk"], final_state=True)
    torch.cuda.synchronize()
    order = np.argsort(lengths)
    for i in sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 7}):
        s, e = int(p["cu_seqlens"][i]), int(p["cu_seqlens"][i + 1])
        yr, fr = oracle.forward(f64(p["x"][None, s:e]), f64(p["log_a"][None, s:e]), f64(p["B"][None, s:e]),
                                f64(p["C"][None, s:e]), f64(p.get("D")), None)
        ey = rel_l2(y[s:e].double().cpu().numpy(), yr[0])
        ef = rel_l2(fin[i].double().cpu().numpy(), fr[0])
        announce("full varlen sequence %d (%d tokens): y %.2e final %.2e" % (i, e - s, ey, ef))
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (i, ey, ef)


@pytest.mark.parametrize("name", ["mamba2_layer", "diag_multiscale", "gqa_decode", "long_seq"])
def test_forward_dt_full_workload(name):
    """ssd_forward_dt over the whole workload as ``bench.py --front-end dt`` runs it (dt and A_log in,
    input scaled, no bias) against the oracle's discretisation and recurrence, every output.  (The
    grouped-heads and long-sequence workloads carry 268 MB of x, which the scalar walk reads with
    streaming loads.)"""
    import oracle.discretize
    cfg = ssd_inputs.config(name)
    announce("full forward_dt %s" % name)
    inp = ssd_inputs.make_inputs(cfg, ssd_inputs.SEEDS[name])
    g = to_gpu(inp)
    y, fin = ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"), chunk=cfg["chunk"],
                                init_state=g.get("init_state"), final_state=True)
    torch.cuda.synchronize()
    yr, fr = oracle.discretize.forward_dt(oracle.default_oracle(), f64(inp["x"]), f64(inp["dt"]), f64(inp["A_log"]),
                                          f64(inp["B"]), f64(inp["C"]), f64(inp.get("D")),
                                          init_state=f64(inp.get("init_state")), diag=cfg["decay"] == "diag")
    ey, ef = rel_l2(y.double().cpu().numpy(), yr), rel_l2(fin.double().cpu().numpy(), fr)
    announce("full forward_dt %s: y %.2e final %.2e" % (name, ey, ef))
    assert ey <= TOL[cfg["dtype"]] and ef <= TOL[cfg["dtype"]]
