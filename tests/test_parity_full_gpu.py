"""Full-size workloads, in the launch configuration the benchmark times, checked against the
oracle on every (batch, head) unit: pooled relL2 over the whole output and the largest relL2 of
any single unit, for y, the SSD part y - D x and the final state (the oracle runs the whole
workload in seconds, so nothing is sampled)."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs
import ssd_chunked_scan_02_amd as ssd
from gpu_helpers import announce, compare_all_units, gpu_forward, per_unit_rel_l2, rel_l2, to_gpu, TOL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_fp32", "mamba2_layer", "long_seq", "gqa_decode", "diag_multiscale"])
def test_full_workload_every_unit(name):
    cfg = ssd_inputs.config(name)
    seed = ssd_inputs.SEEDS[name]
    announce("full %s (seed %d)" % (name, seed))
    inp = ssd_inputs.make_inputs(cfg, seed)
    g = to_gpu(inp)
    y, fin = gpu_forward(g, cfg["chunk"], True)
    compare_all_units(inp, y, fin, cfg["dtype"], "full " + name)


@pytest.mark.parametrize("name", ["mamba2_layer", "long_seq", "gqa_decode", "diag_multiscale"])
def test_full_workload_without_skip_term(name):
    """The same full-size inputs with the skip term removed (D absent): y is then the SSD part
    alone, so the plain bound applies to it pooled and on every unit, with no allowance for the
    output rounding of a D x that dominates y (the launch configuration is the same: the kernels
    add D x with D = 0 when it is absent)."""
    cfg = ssd_inputs.config(name)
    seed = ssd_inputs.SEEDS[name]
    announce("full %s without the skip term (seed %d)" % (name, seed))
    inp = ssd_inputs.make_inputs(cfg, seed)
    inp["D"] = None
    g = to_gpu(inp)
    y, fin = gpu_forward(g, cfg["chunk"], True)
    compare_all_units(inp, y, fin, cfg["dtype"], "full %s, no skip" % name)


def test_decode_continues_forward():
    """gqa_decode: forward over T tokens, then 256 ssd_step calls from its final state, equal
    the oracle run over all T + 256 tokens, for both y and the state, on every (batch, head)."""
    name = "gqa_decode"
    cfg = ssd_inputs.config(name)
    seed = ssd_inputs.SEEDS[name]
    announce("decode after full %s" % name)
    inp = ssd_inputs.make_inputs(cfg, seed)
    g = to_gpu(inp)
    y, state = gpu_forward(g, cfg["chunk"], True)
    steps = cfg["decode_steps"]
    ys = []
    for k in range(steps):
        ys.append(ssd.ssd_step(state, g["x_dec"][:, k].contiguous(), g["log_a_dec"][:, k].contiguous(),
                               g["B_dec"][:, k].contiguous(), g["C_dec"][:, k].contiguous(), g["D"]))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, 1).double().cpu().numpy()
    f = ssd_inputs.to_f64
    whole = {k: torch.cat([inp[k], inp[k + "_dec"]], 1) for k in ("x", "log_a", "B", "C")}
    want_y, want_f = oracle.forward(f(whole["x"]), f(whole["log_a"]), f(whole["B"]), f(whole["C"]), f(inp["D"]),
                                    None)
    T = cfg["seqlen"]
    want_tail = want_y[:, T:]
    got_f = state.double().cpu().numpy()
    tol = TOL["bf16"]
    e_y, e_f = rel_l2(y_dec, want_tail), rel_l2(got_f, want_f)
    uy = per_unit_rel_l2(y_dec, want_tail)
    df = got_f - want_f
    uf = np.sqrt((df ** 2).sum(axis=(2, 3))) / np.sqrt((want_f ** 2).sum(axis=(2, 3)))
    announce("decode 256 steps: relL2 y %.3e final %.3e; max per unit y %.3e final %.3e (tol %.0e)"
             % (e_y, e_f, float(uy.max()), float(uf.max()), tol))
    assert e_y <= tol and e_f <= tol
    assert float(uy.max()) <= tol and float(uf.max()) <= tol
