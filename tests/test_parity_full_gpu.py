"""Full-size workloads, in the launch configuration the benchmark times, checked against the
oracle on sampled (batch, head) units (each head is independent, so the oracle computes
the sampled heads exactly, over the whole sequence)."""
import pytest
import torch

import ssd_inputs
import ssd_chunked_scan_02_amd as ssd
from gpu_helpers import announce, compare, gpu_forward, oracle_forward, to_gpu

pytestmark = pytest.mark.gpu


def _units(cfg, n, seed):
    gen = torch.Generator().manual_seed(seed)
    total = cfg["batch"] * cfg["nheads"]
    picks = torch.randperm(total, generator=gen)[:n].tolist()
    # always include the first and the last unit
    picks = sorted(set(picks) | {0, total - 1})
    return [(u // cfg["nheads"], u % cfg["nheads"]) for u in picks]


@pytest.mark.parametrize("name", ["tiny_fp32", "mamba2_layer", "long_seq", "gqa_decode", "diag_multiscale"])
def test_full_workload_sampled(name):
    cfg = ssd_inputs.config(name)
    seed = ssd_inputs.SEEDS[name]
    announce("full %s (seed %d)" % (name, seed))
    inp = ssd_inputs.make_inputs(cfg, seed)
    g = to_gpu(inp)
    y, fin = gpu_forward(g, cfg["chunk"], True)
    units = None if name == "tiny_fp32" else _units(cfg, 6, seed)
    compare(inp, y, fin, oracle_forward(inp, units), cfg["dtype"], True, "full " + name)


def test_decode_continues_forward():
    """gqa_decode: forward over T tokens, then 256 ssd_step calls from its final state, equal
    the oracle run over all T + 256 tokens (sampled heads), for both y and the state."""
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
    y_dec = torch.stack(ys, 1)
    whole = {k: (torch.cat([inp[k], inp[k + "_dec"]], 1) if k in ("x", "log_a", "B", "C") else v)
             for k, v in inp.items() if not k.endswith("_dec")}
    units = _units(cfg, 4, seed + 1)
    ref = oracle_forward(whole, units)
    T = cfg["seqlen"]
    tail = {k: (v[0][T:], v[1]) for k, v in ref.items()}
    dec_inp = {"x": inp["x_dec"], "D": inp["D"]}
    compare(dec_inp, y_dec, state, tail, "bf16", True, "decode 256 steps")
