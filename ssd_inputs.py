"""Seeded synthetic inputs for the SSD forward workloads.

This module holds only input recipes (shapes, distributions, draw order) and none of the
method's arithmetic; both the CPU oracle's callers and the GPU path's callers use it.

Recipe (all draws on the host from ``torch.Generator('cpu').manual_seed(seed)``, in this
fixed order: x, B, C, dt, A_log, D, init_state; drawn in fp32, then cast to the storage
dtype with round-to-nearest-even):
  x ~ N(0, 1)               [B, T, H, P]
  B, C ~ N(0, 1/N)          [B, T, G, N]     (the second parameter of N(.,.) is a variance)
  dt ~ N(mu, 1)             [B, T, H]        (mu = -2; mu = 0 for the tiny fp32 case)
  A_log                     per head ~ U(0, ln 16), zero for the tiny case, or per state
                            dimension linspace(0, ln 64, N) for the diagonal case (or, in
                            tests, per (head, state dimension) ~ U(0, ln 64))
  log_a = -softplus(dt) * exp(A_log)   in fp32, stored fp32 (the zero-order-hold decay
                            log of exp(Delta*A) with Delta = softplus(dt), A = -exp(A_log))
  D ~ N(0, 1)               [H]              (absent for the tiny case)
  init_state ~ N(0, 0.1)    [B, H, N, P]     fp32 (long-sequence case only)
A decode tail of ``decode_steps`` tokens is drawn together with the prompt (T + steps
tokens) and split off afterwards.  The draws dt and A_log are returned as well (A_log as [H]
for scalar decay, [H, N] for diagonal decay), for the entry points that take them in place of
log_a.
"""
from __future__ import annotations

import math

import torch

# name -> workload.  ``chunk`` is the decomposition's chunk length Q.
CONFIGS = {
    "tiny_fp32": dict(batch=1, seqlen=256, nheads=1, ngroups=1, headdim=64, dstate=16,
                      chunk=64, dtype="fp32", decay="scalar", dt_mean=0.0, a_log="zero",
                      skip=False, init=False, final=False, decode_steps=0),
    "mamba2_layer": dict(batch=8, seqlen=2048, nheads=24, ngroups=1, headdim=64, dstate=128,
                         chunk=128, dtype="bf16", decay="scalar", dt_mean=-2.0,
                         a_log="uniform16", skip=True, init=False, final=False,
                         decode_steps=0),
    "long_seq": dict(batch=1, seqlen=65536, nheads=32, ngroups=1, headdim=64, dstate=128,
                     chunk=256, dtype="bf16", decay="scalar", dt_mean=-2.0,
                     a_log="uniform16", skip=True, init=True, final=True, decode_steps=0),
    "gqa_decode": dict(batch=4, seqlen=8192, nheads=64, ngroups=8, headdim=64, dstate=128,
                       chunk=128, dtype="bf16", decay="scalar", dt_mean=-2.0,
                       a_log="uniform16", skip=True, init=False, final=True,
                       decode_steps=256),
    "diag_multiscale": dict(batch=4, seqlen=4096, nheads=16, ngroups=1, headdim=64,
                            dstate=64, chunk=64, dtype="bf16", decay="diag", dt_mean=-2.0,
                            a_log="linspace64", skip=True, init=False, final=False,
                            decode_steps=0),
}

# Seed of each named workload in the benchmark.
SEEDS = {"tiny_fp32": 1, "mamba2_layer": 2, "long_seq": 3, "gqa_decode": 4, "diag_multiscale": 5}

STORAGE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def config(name: str, **overrides) -> dict:
    """A copy of workload ``name`` with fields replaced by ``overrides``."""
    cfg = dict(CONFIGS[name])
    for k, v in overrides.items():
        if k not in cfg:
            raise KeyError("unknown workload field %r" % k)
        cfg[k] = v
    return cfg


def make_inputs(cfg: dict, seed: int) -> dict:
    """Draw one workload's inputs on the CPU.  Returns a dict of CPU tensors:
    x, log_a, B, C (storage dtypes), D (fp32 [H] or None), init_state (fp32 or None),
    and for decode workloads x_dec, log_a_dec, B_dec, C_dec (one slice per step).
    """
    Bsz, T, H, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["ngroups"]
    P, N = cfg["headdim"], cfg["dstate"]
    steps = cfg.get("decode_steps", 0)
    Tt = T + steps
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    store = STORAGE[cfg["dtype"]]

    x = torch.randn((Bsz, Tt, H, P), generator=gen, dtype=torch.float32)
    Bm = torch.randn((Bsz, Tt, G, N), generator=gen, dtype=torch.float32) / math.sqrt(N)
    Cm = torch.randn((Bsz, Tt, G, N), generator=gen, dtype=torch.float32) / math.sqrt(N)
    dt = torch.randn((Bsz, Tt, H), generator=gen, dtype=torch.float32) + cfg["dt_mean"]
    kind = cfg["a_log"]
    if kind == "zero":
        a_log = torch.zeros(H, dtype=torch.float32)
    elif kind == "uniform16":
        a_log = torch.rand(H, generator=gen, dtype=torch.float32) * math.log(16.0)
    elif kind == "linspace64":
        a_log = torch.linspace(0.0, math.log(64.0), N, dtype=torch.float32)
    elif kind == "rand_hn":
        a_log = torch.rand((H, N), generator=gen, dtype=torch.float32) * math.log(64.0)
    else:
        raise ValueError(kind)
    D = torch.randn(H, generator=gen, dtype=torch.float32) if cfg["skip"] else None
    init = (torch.randn((Bsz, H, N, P), generator=gen, dtype=torch.float32) * math.sqrt(0.1)
            if cfg["init"] else None)

    rate = torch.nn.functional.softplus(dt)
    if cfg["decay"] == "scalar":
        if a_log.shape != (H,):
            raise ValueError("scalar decay needs one A_log per head")
        log_a = -(rate * torch.exp(a_log)[None, None, :])
    else:
        if a_log.shape == (N,):
            a_log = a_log[None, :].expand(H, N)
        elif a_log.shape == (H,):
            a_log = a_log[:, None].expand(H, N)
        log_a = -(rate[..., None] * torch.exp(a_log)[None, None, :, :])
    log_a = log_a.contiguous()

    out = dict(x=x[:, :T].to(store).contiguous(), log_a=log_a[:, :T].contiguous(),
               B=Bm[:, :T].to(store).contiguous(), C=Cm[:, :T].to(store).contiguous(),
               D=D, init_state=init, dt=dt[:, :T].contiguous(), A_log=a_log.contiguous())
    if steps:
        out["x_dec"] = x[:, T:].to(store).contiguous()
        out["log_a_dec"] = log_a[:, T:].contiguous()
        out["dt_dec"] = dt[:, T:].contiguous()
        out["B_dec"] = Bm[:, T:].to(store).contiguous()
        out["C_dec"] = Cm[:, T:].to(store).contiguous()
    return out


def to_f64(t):
    """Exact widening of a stored tensor (fp32 or bf16) to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def dt_bias(nheads: int, seed: int):
    """A step-size bias per head, ~ N(0, 0.25) fp32 [H], from its own generator (seed)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn(nheads, generator=gen, dtype=torch.float32) * 0.5


def output_gradients(cfg: dict, seed: int) -> dict:
    """Seeded dL/dy (N(0,1) in the storage dtype, [B,T,H,P]) and dL/dfinal (N(0,1) fp32
    [B,H,N,P]) for backward-pass workloads, from their own generator."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    Bsz, T, H, P, N = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"]
    dy = torch.randn((Bsz, T, H, P), generator=gen, dtype=torch.float32).to(STORAGE[cfg["dtype"]]).contiguous()
    dfinal = torch.randn((Bsz, H, N, P), generator=gen, dtype=torch.float32)
    return dict(dy=dy, dfinal=dfinal)


def packed_lengths(nseq: int, total: int, seed: int, spread: float = 1.0) -> list:
    """nseq sequence lengths summing to total (each >= 1): a seeded log-normal mix (sigma
    ``spread``) of the kind a serving batch of prompts has, short and long together."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    w = torch.exp(torch.randn(nseq, generator=gen, dtype=torch.float64) * spread)
    raw = (w / w.sum() * (total - nseq)).floor().to(torch.int64) + 1
    raw[int(torch.argmax(raw))] += total - int(raw.sum())
    return [int(v) for v in raw]


def packed_inputs(cfg: dict, lengths, seed: int) -> dict:
    """A packed variable-length batch with the workload's value distributions: the sequences of
    ``lengths`` one after another on one token axis (x [T,H,P], log_a [T,H] or [T,H,N], B, C
    [T,G,N], dt [T,H]), cu_seqlens (int64 [nseq + 1]), max_seqlen, D as the workload's, and with
    cfg["init"] one initial state per sequence ~ N(0, 0.1) [nseq,H,N,P]."""
    lengths = [int(v) for v in lengths]
    total = sum(lengths)
    one = make_inputs(dict(cfg, batch=1, seqlen=total, init=False, decode_steps=0), seed)
    out = {k: (v[0].contiguous() if k in ("x", "log_a", "B", "C", "dt") else v) for k, v in one.items()}
    out.pop("init_state", None)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    out["cu_seqlens"] = cu
    out["max_seqlen"] = max(lengths) if lengths else 0
    out["init_state"] = None
    if cfg["init"]:
        gen = torch.Generator(device="cpu").manual_seed(int(seed) + 7919)
        out["init_state"] = torch.randn((len(lengths), cfg["nheads"], cfg["dstate"], cfg["headdim"]), generator=gen,
                                        dtype=torch.float32) * math.sqrt(0.1)
    return out
