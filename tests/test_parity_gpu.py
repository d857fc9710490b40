"""HIP path against the fp64 oracle, element by element on the same seeded inputs.

Sizes the oracle finishes in seconds that still span several chunks, several 16-token
blocks and a ragged final chunk; the full-size workloads (in the launch configuration the
benchmark times) are checked on sampled (batch, head) units, which the oracle computes one
by one.  Bounds: relative L2 <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs, on y, on
the SSD part y - D x, and on the final state."""
import numpy as np
import pytest
import torch

import ssd_inputs
from gpu_helpers import announce, compare, gpu_forward, oracle_forward, to_gpu, TOL

pytestmark = pytest.mark.gpu


def _run(cfg, seed, label, units=None):
    announce("%s seed=%d cfg=%s" % (label, seed, {k: cfg[k] for k in ("batch", "seqlen", "nheads", "ngroups", "headdim", "dstate", "chunk", "dtype", "decay")}))
    inp = ssd_inputs.make_inputs(cfg, seed)
    g = to_gpu(inp)
    y, fin = gpu_forward(g, cfg["chunk"], True)
    ref = oracle_forward(inp, units)
    return compare(inp, y, fin, ref, cfg["dtype"], True, label)


# ---- reduced versions of the five workloads (several chunks + a ragged tail) -----------
SMALL = [
    ("tiny_fp32", dict()),
    ("tiny_fp32", dict(seqlen=250, skip=True, init=True)),
    ("mamba2_layer", dict(batch=2, seqlen=520, nheads=4)),
    ("long_seq", dict(seqlen=1300, nheads=2)),
    ("gqa_decode", dict(batch=2, seqlen=700, nheads=8, ngroups=2, decode_steps=0)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=["%s-%d" % (n, i) for i, (n, _) in enumerate(SMALL)])
def test_small_workloads(name, over):
    cfg = ssd_inputs.config(name, **over)
    _run(cfg, 7, "small " + name)


SEGMENTED = [
    # few (batch, head) units on a long sequence: the walk runs in segments (state-only pass,
    # prefix over segment states, full pass from each segment's start state)
    dict(batch=1, seqlen=3000, nheads=2, chunk=128, init=True),
    dict(batch=2, seqlen=2100, nheads=4, ngroups=2, chunk=64, init=True, skip=False),
    dict(batch=1, seqlen=4100, nheads=1, chunk=256, dstate=64),
    # slow decay (softplus(dt) ~ 3e-4): every chunk of a segment weighs in the segment state
    dict(batch=1, seqlen=3000, nheads=2, chunk=128, init=True, dt_mean=-8.0),
    # fast decay: the segment state pass stops after the last chunk or two, since every earlier
    # token's weight is 0 in fp32
    dict(batch=1, seqlen=3000, nheads=2, chunk=128, init=True, dt_mean=2.0),
]


@pytest.mark.parametrize("over", SEGMENTED, ids=["seg-%d" % i for i in range(len(SEGMENTED))])
def test_segmented_walk(over):
    cfg = ssd_inputs.config("mamba2_layer", **over)
    _run(cfg, 23, "segmented")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_chunk_sizes(dtype, chunk):
    """Every supported chunk length gives the oracle's result (the decomposition is exact)."""
    cfg = ssd_inputs.config("mamba2_layer", batch=1, seqlen=600, nheads=3, dstate=64,
                            chunk=chunk, dtype=dtype, init=True)
    _run(cfg, 11, "chunk=%d %s" % (chunk, dtype))


@pytest.mark.parametrize("dtype,N,P", [("bf16", 32, 32), ("bf16", 64, 128), ("bf16", 256, 64),
                                       ("bf16", 128, 16), ("fp32", 16, 64), ("fp32", 64, 32),
                                       ("fp32", 128, 64)])
def test_state_and_head_dims(dtype, N, P):
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=300, nheads=2, dstate=N, headdim=P,
                            chunk=64, dtype=dtype, init=True)
    _run(cfg, 13, "N=%d P=%d %s" % (N, P, dtype))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_one_head_per_group(dtype):
    """H = G: every head has its own B and C (no sharing of the score tiles)."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=333, nheads=3, ngroups=3, dtype=dtype, init=True)
    _run(cfg, 61, "H=G %s" % dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_no_skip_term(dtype):
    """D absent: the whole output is the SSD part, so no skip term can mask an error."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=400, nheads=3, dtype=dtype, skip=False)
    _run(cfg, 17, "no skip %s" % dtype)


@pytest.mark.parametrize("seqlen", [1, 15, 16, 17, 127, 129])
def test_short_and_ragged_sequences(seqlen):
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=seqlen, nheads=2, init=True)
    _run(cfg, 19, "T=%d" % seqlen)


def test_empty_sequence_returns_initial_state():
    announce("T=0")
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=0, nheads=2, init=True)
    inp = ssd_inputs.make_inputs(cfg, 3)
    g = to_gpu(inp)
    y, fin = gpu_forward(g, cfg["chunk"], True)
    assert y.shape[1] == 0
    assert torch.equal(fin.cpu(), inp["init_state"])
    g["init_state"] = None
    y, fin = gpu_forward(g, cfg["chunk"], True)
    assert torch.count_nonzero(fin).item() == 0


def test_empty_batch():
    announce("batch=0")
    cfg = ssd_inputs.config("mamba2_layer", batch=0, seqlen=64, nheads=2)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 3))
    y, fin = gpu_forward(g, cfg["chunk"], True)
    assert y.numel() == 0 and fin.numel() == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_closed_form_decays(dtype):
    """a = 1 (log a = 0) and a = 0 (log a = -1e4) on the GPU against the oracle."""
    for value, label in ((0.0, "a=1"), (-1e4, "a=0")):
        cfg = ssd_inputs.config("mamba2_layer", batch=1, seqlen=300, nheads=2, dtype=dtype, init=True)
        inp = ssd_inputs.make_inputs(cfg, 23)
        inp["log_a"] = torch.full_like(inp["log_a"], value)
        announce("%s %s" % (label, dtype))
        y, fin = gpu_forward(to_gpu(inp), cfg["chunk"], True)
        compare(inp, y, fin, oracle_forward(inp), dtype, True, "%s %s" % (label, dtype))


def test_extreme_decays_stay_finite():
    """Very fast decays (down to -1e4 per step) and mixed rates: finite and within bounds."""
    cfg = ssd_inputs.config("mamba2_layer", batch=1, seqlen=512, nheads=4, init=True)
    inp = ssd_inputs.make_inputs(cfg, 29)
    gen = torch.Generator().manual_seed(5)
    mult = torch.exp(torch.rand(inp["log_a"].shape, generator=gen) * 12.0)   # up to e^12 faster
    inp["log_a"] = torch.clamp(inp["log_a"] * mult, min=-1e4).contiguous()
    announce("extreme decays")
    y, fin = gpu_forward(to_gpu(inp), cfg["chunk"], True)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    compare(inp, y, fin, oracle_forward(inp), "bf16", True, "extreme decays")


def test_deterministic_and_writes_every_output():
    """Bitwise identical across runs; outputs prefilled with NaN are all overwritten."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=333, nheads=3, init=True)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 31))
    announce("determinism / NaN poisoning")
    outs = []
    for _ in range(3):
        y = torch.full((2, 333, 3, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        fin = torch.full((2, 3, 128, 64), float("nan"), dtype=torch.float32, device="cuda")
        import ssd_chunked_scan_02_amd as ssd
        ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g["D"], chunk=cfg["chunk"],
                        init_state=g["init_state"], y=y, final_state=fin)
        torch.cuda.synchronize()
        assert not torch.isnan(y.float()).any() and not torch.isnan(fin).any()
        outs.append((y.cpu(), fin.cpu()))
    for y, fin in outs[1:]:
        assert torch.equal(y.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(fin, outs[0][1])


@pytest.mark.parametrize("over,launches", [(dict(batch=2, seqlen=333, nheads=3), 2),
                                            (dict(batch=1, seqlen=3000, nheads=2, init=True), 3)],
                         ids=["whole", "segmented"])
def test_profiled_forward_times_each_launch(over, launches):
    """ssd_forward_profiled: every launch stamps its own start/end event pair, the run times are
    positive, and the outputs are bitwise those of ssd_forward."""
    import ssd_chunked_scan_02_amd as ssd
    from bench import HipEvents
    cfg = ssd_inputs.config("mamba2_layer", **over)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 37))
    announce("profiled forward %s" % over)
    kw = dict(chunk=cfg["chunk"], init_state=g.get("init_state"), final_state=True)
    y0, f0 = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), **kw)
    ev = HipEvents()
    events = [ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)]
    try:
        y1, f1, n = ssd.ssd_forward_profiled(g["x"], g["log_a"], g["B"], g["C"], g.get("D"),
                                             events=events, **kw)
        torch.cuda.synchronize()
        assert n == launches
        times = [ev.elapsed_ms(events[2 * k], events[2 * k + 1]) for k in range(n)]
        assert all(0.0 < t < 1000.0 for t in times), times
    finally:
        for e in events:
            ev.destroy(e)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)) and torch.equal(f0, f1)


def test_split_resume_matches_whole():
    """forward(T1) then forward(T2, init = final1) equals forward(T1 + T2) (chunk-aligned and
    not), up to the bf16 rounding of y."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=700, nheads=3, init=True)
    inp = ssd_inputs.make_inputs(cfg, 37)
    g = to_gpu(inp)
    announce("split/resume")
    y, fin = gpu_forward(g, 128, True)
    for t1 in (256, 301):
        a = {k: (v[:, :t1].contiguous() if k in ("x", "log_a", "B", "C") else v) for k, v in g.items()}
        ya, fa = gpu_forward(a, 128, True)
        bpart = {k: (v[:, t1:].contiguous() if k in ("x", "log_a", "B", "C") else v) for k, v in g.items()}
        bpart["init_state"] = fa
        yb, fb = gpu_forward(bpart, 128, True)
        e = (torch.cat([ya, yb], 1).float() - y.float()).norm() / y.float().norm()
        ef = (fb - fin).norm() / fin.norm()
        announce("split at %d: relL2 y %.2e final %.2e" % (t1, e, ef))
        assert e < 1e-2 and ef < 1e-4


# ---- diagonal (per-state-dimension) decay -----------------------------------------------
DIAG_SMALL = [
    dict(batch=2, seqlen=300, nheads=4),                                   # ragged tail
    dict(batch=1, seqlen=256, nheads=2, dstate=128, headdim=32),
    dict(batch=2, seqlen=200, nheads=2, dtype="fp32", dstate=32, headdim=32, chunk=32),
    dict(batch=1, seqlen=190, nheads=3, dtype="fp32", dstate=64, headdim=64, init=True),
]


@pytest.mark.parametrize("over", DIAG_SMALL, ids=lambda o: "-".join("%s%s" % kv for kv in o.items()))
def test_diag_small(over):
    cfg = ssd_inputs.config("diag_multiscale", **over)
    _run(cfg, 41, "diag")


DIAG_SEGMENTED = [
    # few units on a long sequence: state-only pass, per-row segment prefix, full pass
    dict(batch=1, seqlen=2000, nheads=2, init=True),
    dict(batch=2, seqlen=1100, nheads=1, dstate=32, headdim=32, skip=False),
]


@pytest.mark.parametrize("over", DIAG_SEGMENTED, ids=["diag-seg-%d" % i for i in range(len(DIAG_SEGMENTED))])
def test_diag_segmented(over):
    cfg = ssd_inputs.config("diag_multiscale", **over)
    _run(cfg, 59, "diag segmented")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_diag_chunk_sizes(chunk):
    cfg = ssd_inputs.config("diag_multiscale", batch=1, seqlen=333, nheads=2, chunk=chunk, init=True)
    _run(cfg, 43, "diag chunk=%d" % chunk)


def test_diag_equal_rates_match_scalar_oracle():
    """A per-dimension decay that is the same for every n is the scalar-decay model."""
    cfg = ssd_inputs.config("mamba2_layer", batch=2, seqlen=300, nheads=3, dstate=64, chunk=64, init=True)
    inp = ssd_inputs.make_inputs(cfg, 47)
    announce("diag with equal rates vs scalar oracle")
    ref = oracle_forward(inp)
    diag = dict(inp)
    diag["log_a"] = inp["log_a"][..., None].expand(-1, -1, -1, 64).contiguous()
    y, fin = gpu_forward(to_gpu(diag), 64, True)
    compare(inp, y, fin, ref, "bf16", True, "diag equal rates")


def test_diag_extreme_rates():
    """Per-dimension steps down to -1e4 (the state dimension forgets within one token)."""
    cfg = ssd_inputs.config("diag_multiscale", batch=1, seqlen=256, nheads=2, init=True)
    inp = ssd_inputs.make_inputs(cfg, 53)
    gen = torch.Generator().manual_seed(7)
    mult = torch.exp(torch.rand(inp["log_a"].shape, generator=gen) * 8.0)
    inp["log_a"] = torch.clamp(inp["log_a"] * mult, min=-1e4).contiguous()
    announce("diag extreme rates")
    y, fin = gpu_forward(to_gpu(inp), 64, True)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    compare(inp, y, fin, oracle_forward(inp), "bf16", True, "diag extreme rates")


@pytest.mark.parametrize("scale", [0.02, 4000.0], ids=["small-BC", "large-BC"])
def test_diag_split_bound_magnitudes(scale):
    """B and C entries far from unit size (times 0.02: typical magnitude 2.5e-3; times 4000: up
    to a few thousand) on decays of 6.5 to 10 nats per token, so that every dimension's decay over
    a 16-token block lies near the split bound of the diagonal score tiles (up to 160 nats, each
    factor within e^+-80): the split factors times B and C stay finite and normal there."""
    cfg = ssd_inputs.config("diag_multiscale", batch=1, seqlen=256, nheads=2, init=True)
    inp = ssd_inputs.make_inputs(cfg, 57)
    gen = torch.Generator().manual_seed(11)
    inp["log_a"] = (-(6.5 + 3.5 * torch.rand(inp["log_a"].shape, generator=gen))).to(torch.float32).contiguous()
    for k in ("B", "C"):
        inp[k] = (inp[k].float() * scale).to(inp[k].dtype)
    announce("diag split-bound magnitudes scale=%g" % scale)
    y, fin = gpu_forward(to_gpu(inp), 64, True)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    compare(inp, y, fin, oracle_forward(inp), "bf16", True, "diag split-bound magnitudes x%g" % scale)


def test_decode_steps_in_a_hip_graph():
    """ssd_step launches captured in a HIP graph (as the decode timing replays them) give the
    eager result bitwise, on every one of several replays with eager work in between."""
    import ssd_chunked_scan_02_amd as ssd
    cfg = ssd_inputs.config("gqa_decode", batch=2, seqlen=64, nheads=8, ngroups=2, decode_steps=6,
                            final=True)
    g = to_gpu(ssd_inputs.make_inputs(cfg, 43))
    announce("decode steps in a HIP graph")
    _, s0 = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g["D"], chunk=cfg["chunk"],
                            final_state=True)
    steps = [tuple(g[k][:, i].contiguous() for k in ("x_dec", "log_a_dec", "B_dec", "C_dec"))
             for i in range(cfg["decode_steps"])]
    cap = torch.cuda.Stream()
    state = s0.clone()
    ys = [torch.empty((2, 8, 64), dtype=torch.bfloat16, device="cuda") for _ in steps]

    def run(st):
        for (x, la, bb, cc), y in zip(steps, ys):
            ssd.ssd_step(st, x, la, bb, cc, D=g["D"], y_t=y, stream=cap)

    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        run(state)
    torch.cuda.synchronize()
    want_state, want_y = state.clone(), [y.clone() for y in ys]
    graph = torch.cuda.CUDAGraph()
    state.copy_(s0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        run(state)
    for rep in range(3):
        state.copy_(s0)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, want_state), rep
        for y, w in zip(ys, want_y):
            assert torch.equal(y.view(torch.int16), w.view(torch.int16)), rep


def test_side_stream_call_keeps_its_memory():
    """A call on a side stream whose workspace and outputs the binding allocates: right after it
    returns (its kernels still running), same-sized allocations on torch's current stream are
    filled with NaN.  The allocator must not hand them the call's memory before its kernels end,
    so the outputs equal those of a call on the current stream bit for bit."""
    import ssd_chunked_scan_02_amd as ssd
    cfg = ssd_inputs.config("mamba2_layer")
    g = to_gpu(ssd_inputs.make_inputs(cfg, 211))
    announce("side-stream call with allocations on the current stream")
    y0, _ = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g["D"], chunk=cfg["chunk"])
    torch.cuda.synchronize()
    dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
    ws_bytes = ssd.ssd_forward_workspace_bytes(dims, cfg["chunk"])
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        y, _ = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g["D"], chunk=cfg["chunk"], stream=side)
        junk = [torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda"),
                torch.full(tuple(y.shape), float("nan"), dtype=y.dtype, device="cuda")]
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), rep
        del junk


# (bf16 covers N 32..256, fp32 N 16..128; rows per thread 1, 2, 4, 8 and 16)
STEP_SHAPES = [("bf16", "scalar", 32, 16), ("bf16", "scalar", 256, 64), ("bf16", "scalar", 128, 128),
               ("bf16", "diag", 32, 32), ("fp32", "scalar", 128, 128), ("fp32", "diag", 16, 64),
               ("fp32", "scalar", 64, 16), ("bf16", "diag", 256, 32), ("fp32", "diag", 64, 64),
               ("bf16", "scalar", 32, 64)]


@pytest.mark.parametrize("dtype,decay,N,P", STEP_SHAPES, ids=["%s-%s-n%d-p%d" % s for s in STEP_SHAPES])
def test_step_shapes_continue_forward(dtype, decay, N, P):
    """Decode steps at every rows-per-thread split of the step kernel (state dims 16..256, head
    dims 16..128, both element types and both decay kinds): k steps from an initial state equal
    the oracle's recurrence over the same k tokens, y of every step and the final state."""
    import oracle
    import ssd_chunked_scan_02_amd as ssd
    from gpu_helpers import rel_l2
    name = "diag_multiscale" if decay == "diag" else "mamba2_layer"
    cfg = ssd_inputs.config(name, batch=2, seqlen=1, nheads=4, ngroups=2, dstate=N, headdim=P, dtype=dtype,
                            init=True, decode_steps=9)
    inp = ssd_inputs.make_inputs(cfg, 223)
    g = to_gpu(inp)
    announce("step shapes %s %s N=%d P=%d" % (dtype, decay, N, P))
    state = g["init_state"].clone()
    ys = [ssd.ssd_step(state, g["x_dec"][:, t].contiguous(), g["log_a_dec"][:, t].contiguous(),
                       g["B_dec"][:, t].contiguous(), g["C_dec"][:, t].contiguous(), g["D"]).clone()
          for t in range(cfg["decode_steps"])]
    torch.cuda.synchronize()
    f = ssd_inputs.to_f64
    yr, fr = oracle.forward(f(inp["x_dec"]), f(inp["log_a_dec"]), f(inp["B_dec"]), f(inp["C_dec"]), f(inp["D"]),
                            f(inp["init_state"]))
    y_dec = np.stack([y.double().cpu().numpy() for y in ys], 1)
    e_y = rel_l2(y_dec, yr)
    e_f = rel_l2(state.double().cpu().numpy(), fr)
    announce("step shapes %s %s N=%d P=%d: y %.2e final %.2e" % (dtype, decay, N, P, e_y, e_f))
    assert e_y <= TOL[dtype] and e_f <= TOL[dtype]
