#!/usr/bin/env python3
"""Benchmark of the chunked SSD forward on one MI355X.

Prints ONE JSON line on stdout: tokens/s of ssd_forward on the Mamba-2 layer workload
(B=8, T=2048, H=24, G=1, P=64, N=128, chunk 128, bf16 x/B/C/y, fp32 log a, D and state),
with TFLOP/s, fraction of MFMA peak, the HBM roofline of the dominant kernel (timed live
with HIP events that each launch's dispatch stamps at its start and end, on the launch
stream) and the fp64 CPU oracle's throughput on this host as a reported baseline.

A step is one ssd_forward over one batch (with --front-end dt, one ssd_forward_dt: log a and
the input scale formed in the kernels from dt and A_log, the Mamba-2 layer's form).  Inputs are drawn once (seeded, synthetic) and
copied to HBM before timing; the timed steps cycle through several copies of the inputs
and outputs (about 1 GB together) so that no step finds its data in the 256 MB
last-level cache.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "ssd_chunked_scan_02_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_counts(cfg, front_end="log_a"):
    """Work the method must do for one forward over the workload (not what a kernel
    executes): causal C B^T and (S o L) X inside chunks, plus the chunk-state and carried-
    state contractions; bytes = every input read once and every output written once (with the
    dt front-end the decay input is dt [B,T,H] and A_log [H] or [H,N] instead of log a)."""
    Bsz, T, H, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["ngroups"]
    P, N, Q = cfg["headdim"], cfg["dstate"], cfg["chunk"]
    diag = cfg["decay"] == "diag"
    Gs = H if diag else G
    K = N if diag else 1
    sx = 4 if cfg["dtype"] == "fp32" else 2
    flops = Bsz * T * (Gs * N * (Q + 1) + H * P * (Q + 1) + 4 * H * N * P)
    dt = front_end == "dt"
    per_token = H * P * (sx + sx) + 2 * G * N * sx + 4 * H * (1 if dt else K)
    nbytes = Bsz * T * per_token + (4 * H if cfg["skip"] else 0) + (4 * H * K if dt else 0) \
        + 4 * Bsz * H * N * P * (int(cfg["init"]) + int(cfg["final"]))
    return flops, nbytes, per_token


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        h = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return float(out.value)

    def destroy(self, h):
        self.lib.hipEventDestroy(ctypes.c_void_p(h))


# the source file each kernel (by name prefix) and its launch code are compiled from
KERNEL_SOURCES = {"prep_kernel": "ssd_fast.hip", "walk_fast_kernel": "ssd_fast.hip", "mark_tokens_kernel": "ssd_fast.hip",
                  "seg_state_kernel": "ssd_fast.hip", "seg_prefix_kernel": "ssd_fast.hip",
                  "walk_diag_pipe_kernel": "ssd_diag.hip", "walk_diag_kernel": "ssd_diag.hip",
                  "seg_state_diag_kernel": "ssd_diag.hip",
                  "scores_kernel": "ssd_kernels.hip", "walk_kernel": "ssd_kernels.hip",
                  "step_kernel": "ssd_kernels.hip", "discretize_kernel": "ssd_kernels.hip",
                  "skip_kernel": "ssd_kernels.hip", "bwd_states_kernel": "ssd_bwd.hip",
                  "bwd_walk_kernel": "ssd_bwd.hip", "zero_kernel": "ssd_bwd.hip", "bwd_reduce_kernel": "ssd_bwd.hip",
                  "bwd_states_bf16_kernel": "ssd_bwd.hip", "bwd_walk_bf16_kernel": "ssd_bwd.hip",
                  "bwd_local_diag_kernel": "ssd_bwd.hip", "bwd_scan_diag_kernel": "ssd_bwd.hip",
                  "bwd_terms_diag_kernel": "ssd_bwd.hip"}


def _included_headers(name, seen):
    """The headers of csrc that source `name` includes, directly or through other headers."""
    for line in open(os.path.join(CSRC, name)):
        line = line.strip()
        if line.startswith("#include \""):
            inc = line.split("\"")[1]
            if inc not in seen and os.path.exists(os.path.join(CSRC, inc)):
                seen.add(inc)
                _included_headers(inc, seen)
    return seen


def kernel_source_hash(kernel):
    """Hash of the sources `kernel` is built from (its .hip file and the headers it includes):
    counter figures taken on other sources are stale."""
    src = KERNEL_SOURCES[kernel.split("<")[0]]
    names = [src] + sorted(_included_headers(src, set()))
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def fast_segments(cfg, target=256, chunks_per_segment=False):
    """Segments the library splits each (batch, head) sequence into (mirrors its workspace
    layout: only with at most 128 units; about `target` (256) workgroups and at least 4 chunks
    per segment), or with chunks_per_segment the chunks of each segment."""
    q = min(cfg["chunk"], 128)
    units = cfg["batch"] * cfg["nheads"]
    nch = -(-cfg["seqlen"] // q)
    nseg = 1
    if units > 0 and units * 2 <= 256 and nch >= 8:
        nseg = min(target // units, nch // 4)
    per = -(-nch // nseg)
    return per if chunks_per_segment else -(-nch // per)


def packed_as_one(cfg, nseq, tokens):
    """Whether the library walks a packed batch of nseq sequences (tokens in all, lengths bounded
    by cfg["seqlen"]) with no per-sequence states as one sequence (mirrors its estimate: one
    segment's chunks x 1.35 + 2 against the longest sequence's chunks or all (sequence, head)
    chunks over 256 CUs, whichever is more)."""
    q = min(cfg["chunk"], 128)
    nch = -(-tokens // q)
    per = fast_segments(dict(cfg, batch=1, seqlen=tokens), chunks_per_segment=True)
    longest = -(-cfg["seqlen"] // q)
    spread = math.ceil((nch + nseq) * cfg["nheads"] / 256.0)
    return 1.35 * per + 2.0 < max(longest, spread)


def kernel_names(cfg, front_end="log_a", segmented=True, packed=0, tokens=0):
    """Kernels one forward launches, in order (mirrors the library's dispatch).  A packed
    variable-length batch of `packed` sequences (`tokens` in all) with per-sequence states is walked
    sequence by sequence, never segmented, and on the fast path up to 4096 of them are first ranked
    by length; without states the fast path walks it as one sequence of all its tokens (segmented
    as such), with the tokens where each sequence starts marked by the prep kernel (by a launch
    of their own beyond 4095 sequences)."""
    Q, N, P = cfg["chunk"], cfg["dstate"], cfg["headdim"]
    fast = cfg["decay"] != "diag" and cfg["dtype"] == "bf16" and P == 64 and N in (64, 128) and Q in (64, 128, 256)
    if packed and fast and not cfg["init"] and not cfg["final"] and packed_as_one(cfg, packed, tokens):
        marking = ["mark_tokens_kernel"] if packed + 1 > 4096 else []
        return marking + kernel_names(dict(cfg, batch=1, seqlen=tokens), front_end)
    if front_end == "dt":
        fused = (cfg["dtype"] == "bf16" and Q == 64 and N in (32, 64) and P in (32, 64)) if cfg["decay"] == "diag" \
            else (cfg["dtype"] == "bf16" and P == 64 and N in (64, 128) and Q in (64, 128, 256))
        if not fused:
            return ["discretize_kernel"] + kernel_names(cfg) + (["skip_kernel"] if cfg["skip"] else [])
    if cfg["decay"] == "diag":
        if cfg["dtype"] == "bf16" and Q == 64 and N in (32, 64) and P in (32, 64):
            nseg = fast_segments(dict(cfg, chunk=64), 256) if segmented else 1
            if nseg > 1:
                # (up to 4 segments the walk chains the segment states itself)
                prefix = ["seg_prefix_kernel"] if nseg > 4 else []
                return ["seg_state_diag_kernel<%d,%d>" % (N, P)] + prefix + ["walk_diag_pipe_kernel<%d,%d>" % (N, P)]
            return ["walk_diag_pipe_kernel<%d,%d>" % (N, P)]
        return ["walk_diag_kernel<%d,%d>" % (N, P)]
    if cfg["dtype"] == "bf16" and P == 64 and N in (64, 128) and Q in (64, 128, 256):
        q = min(Q, 128)
        if segmented and fast_segments(cfg) > 1:
            return ["prep_kernel<%d,%d>" % (N, q), "seg_state_kernel<%d,%d>" % (N, q),
                    "walk_fast_kernel<%d,%d>" % (N, q)]
        return ["prep_kernel<%d,%d>" % (N, q), "walk_fast_kernel<%d,%d>" % (N, q)]
    return ["scores_kernel<%d>" % N, "walk_kernel<%d,%d>" % (N, P)]


def kernel_bytes(cfg, name, nbytes):
    """Algorithmic bytes of one launch of `name`: what of the method's inputs and outputs that
    kernel itself moves.  The fast path's walk reads x and log a and writes y (B and C reach
    it through the prep kernel); every other walk moves the whole forward's bytes."""
    if not name.startswith("walk_fast_kernel"):
        return nbytes
    Bsz, T, H, N, P = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["dstate"], cfg["headdim"]
    return Bsz * T * (H * P * 4 + 4 * H) + (4 * H if cfg["skip"] else 0) \
        + 4 * Bsz * H * N * P * (int(cfg["init"]) + int(cfg["final"]))


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none or it was taken on different kernel sources."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel.split("<")[0], workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, cfg, min_seconds, front_end="log_a"):
    """The fp64 oracle as it stands, on this host's cores, over the whole workload, repeated
    until at least ``min_seconds`` of CPU wall time (with the dt front-end, the oracle's
    discretisation followed by its recurrence)."""
    import oracle
    import oracle.discretize
    import ssd_inputs
    f = ssd_inputs.to_f64
    args = [f(inp["x"]), f(inp["log_a"]), f(inp["B"]), f(inp["C"]), f(inp.get("D")),
            f(inp.get("init_state"))]
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        if front_end == "dt":
            out = oracle.discretize.forward_dt(oracle.default_oracle(), args[0], f(inp["dt"]), f(inp["A_log"]),
                                               args[2], args[3], args[4], init_state=args[5], want_final=True,
                                               diag=cfg["decay"] == "diag", nthreads=threads)
        else:
            out = oracle.forward(*args, want_final=True, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds and reps >= 1:
            break
    tokens = cfg["batch"] * cfg["seqlen"] * reps
    return ({"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
             "sample": "the whole workload (%d x %d tokens x %d heads), %d run(s) in %.1f s, "
                       "fp64 sequential recurrence, OpenMP over (batch, head)"
                       % (cfg["batch"], cfg["seqlen"], cfg["nheads"], reps, el)}, out)


def output_parity(cfg, inp, y, final, ref):
    """The timed run's outputs against the oracle's on the same stored inputs: relative L2 of y,
    of the SSD part y - D x and of the final state, with the bounds of the parity tests (1e-5
    for fp32 inputs, 2e-2 for bf16; the SSD part's bound adds the one rounding of y, relative to
    the whole of y, that it cannot avoid)."""
    import numpy as np
    import ssd_inputs
    tol = 1e-5 if cfg["dtype"] == "fp32" else 2e-2
    u = 2.0 ** -24 if cfg["dtype"] == "fp32" else 2.0 ** -8
    yr, fr = ref
    yg = y.double().cpu().numpy()
    x = ssd_inputs.to_f64(inp["x"])
    D = ssd_inputs.to_f64(inp.get("D"))
    skip = np.zeros_like(x) if D is None else D[None, None, :, None] * x

    def rel(a, b):
        n = float(np.linalg.norm((b).ravel()))
        return float(np.linalg.norm((a - b).ravel())) / n if n > 0 else float(np.linalg.norm(a.ravel()))

    e_y = rel(yg, yr)
    e_ssd = rel(yg - skip, yr - skip)
    ssd_norm = float(np.linalg.norm((yr - skip).ravel()))
    tol_ssd = tol + (u * float(np.linalg.norm(yr.ravel())) / ssd_norm if ssd_norm > 0 else 0.0)
    out = {"rel_l2_y": e_y, "rel_l2_ssd_part": e_ssd, "tol": tol, "tol_ssd_part": tol_ssd,
           "reference": "fp64 oracle on the same stored inputs; outputs of the timed run"}
    ok = e_y <= tol and e_ssd <= tol_ssd and bool(np.isfinite(yg).all())
    if final is not None and fr is not None:
        out["rel_l2_final"] = rel(final.double().cpu().numpy(), fr)
        ok = ok and out["rel_l2_final"] <= tol
    out["pass"] = bool(ok)
    return out


def backward_parity(cfg, got, want):
    """The timed run's gradients of batch element 0 against the fp64 adjoint's on the same stored
    inputs (the cpu_baseline leg's result): relative L2 of dx, dlog a, dB, dC and dinit, with the
    bounds of the parity tests (1e-5 for fp32 inputs, 2e-2 for bf16).  (dD sums over the batch, so
    it is left to the tests.)"""
    import numpy as np
    tol = 1e-5 if cfg["dtype"] == "fp32" else 2e-2
    out, ok = {}, True
    for k in ("dx", "dlog_a", "dB", "dC", "dinit"):
        if got.get(k) is None or want.get(k) is None:
            continue
        a = got[k][:1].double().cpu().numpy()
        b = np.asarray(want[k])
        n = float(np.linalg.norm(b.ravel()))
        e = float(np.linalg.norm((a - b).ravel())) / n if n > 0 else float(np.linalg.norm(a.ravel()))
        out["rel_l2_" + k] = e
        ok = ok and e <= tol and bool(np.isfinite(a).all())
    out["tol"] = tol
    out["reference"] = "fp64 adjoint on batch element 0 of the same stored inputs; gradients of the timed run"
    out["pass"] = bool(ok)
    return out


def time_decode(ssd, cfg, g, stream, ev, dev):
    """The workload's decode tail: ssd_step for each of its decode tokens, continuing from the
    forward's final state.  The steps are captured once in a HIP graph (their launches would
    otherwise be paced by the host) and one replay is timed with events on the launch stream."""
    import ctypes
    import torch
    steps = cfg["decode_steps"]
    Bsz, H, N, P = cfg["batch"], cfg["nheads"], cfg["dstate"], cfg["headdim"]
    state = g["final"].clone()
    y_t = torch.empty((Bsz, H, P), dtype=g["x"].dtype, device=dev)
    sl = [tuple(g[k][:, i].contiguous() for k in ("x_dec", "log_a_dec", "B_dec", "C_dec"))
          for i in range(steps)]
    lib = ssd.load_library()
    dims = ssd.Dims(Bsz, 1, H, cfg["ngroups"], P, N, ssd.SSD_BF16 if cfg["dtype"] == "bf16" else ssd.SSD_F32,
                    ssd.SSD_DECAY_SCALAR if cfg["decay"] == "scalar" else ssd.SSD_DECAY_DIAG)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    args = [(ctypes.byref(dims), ssd._ptr(state), *(ssd._ptr(t) for t in s4), ssd._ptr(g.get("D")),
             ssd._ptr(y_t), ctypes.c_void_p(cap.cuda_stream)) for s4 in sl]

    def run():
        for a in args:
            if lib.ssd_step(*a) != 0:
                raise RuntimeError("ssd_step failed")

    with torch.cuda.stream(cap):
        run()  # eager once (the library's first call on a device does its set-up outside capture)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        run()
    # torch replays a graph on its current stream: replay on `cap`, where the events are recorded
    with torch.cuda.stream(cap):
        graph.replay()
    torch.cuda.synchronize()
    reps = 5
    b, e = ev.create(), ev.create()
    ev.lib.hipEventRecord(b, cap.cuda_stream)
    with torch.cuda.stream(cap):
        for _ in range(reps):
            graph.replay()
    ev.lib.hipEventRecord(e, cap.cuda_stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(b, e) * 1e3 / (steps * reps)
    ev.destroy(b)
    ev.destroy(e)
    esz = 2 if cfg["dtype"] == "bf16" else 4
    # per step: the fp32 state read and written once, plus x, y, B, C, log a of one token
    state_bytes = 2 * Bsz * H * N * P * 4
    io_bytes = Bsz * H * P * esz * 2 + 2 * Bsz * cfg["ngroups"] * N * esz + Bsz * H * 4
    log("decode: %d steps, %.2f us/step" % (steps, us))
    # (each (batch, head) state lands on the same XCD every step, so it stays in that XCD's L2:
    # the effective rate is not bounded by HBM)
    return {"steps": steps, "us_per_step": us,
            "timing": "%d replays of a HIP graph of all steps, events on the replay stream" % reps,
            "bytes_per_step": state_bytes + io_bytes,
            "effective_gbs": (state_bytes + io_bytes) / (us / 1e6) / 1e9}


def calibrate_copy(dev, mib):
    """A plain streaming kernel of known traffic for the counter calibration: torch's elementwise
    negation reads and writes `mib` MiB each."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    torch.cuda.synchronize()
    dst = torch.neg(src)
    torch.cuda.synchronize()
    del dst
    log("calibration: neg kernel reading and writing %d MiB each" % mib)


def measured_copy_gbs(dev, ev, stream, mib=1024, reps=5):
    """HBM bandwidth this GPU reaches in a plain device copy of `mib` MiB (read once, written
    once), timed with events on the launch stream: the practical ceiling beside the published
    8 TB/s."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    b, e = ev.create(), ev.create()
    ev.lib.hipEventRecord(b, stream.cuda_stream)
    for _ in range(reps):
        dst.copy_(src)
    ev.lib.hipEventRecord(e, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(b, e) / reps
    ev.destroy(b)
    ev.destroy(e)
    del src, dst
    gbs = 2.0 * n / (ms / 1e3) / 1e9
    log("device copy of %d MiB: %.1f GB/s (read + write)" % (mib, gbs))
    return gbs


def shape_text(cfg):
    """The workload's shape as the metric names it: B, T, H, P, N (and G, chunk and the decay
    kind where they differ from one group, chunk 128 and scalar decay)."""
    t = "B=%d,T=%d,H=%d,P=%d,N=%d" % (cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"])
    if cfg["ngroups"] != 1:
        t += ",G=%d" % cfg["ngroups"]
    if cfg["chunk"] != 128:
        t += ",chunk=%d" % cfg["chunk"]
    if cfg["decay"] != "scalar":
        t += ",%s decay" % cfg["decay"]
    if cfg["dtype"] != "bf16":
        t += ",%s" % cfg["dtype"]
    return t


def provenance(workload, seed):
    """Where the numbers come from: the seed, the sources' hash (and the git commit when a
    checkout is present), the GPU and the ROCm / torch versions."""
    import subprocess
    import torch
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.abspath(__file__), "rb") as f:
        h.update(f.read())
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        head = None
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"workload": workload, "seed": seed, "sources_sha256_16": h.hexdigest()[:16], "git_head": head,
            "gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "rocm": rocm, "hip": torch.version.hip, "torch": torch.__version__}


BWD_CHUNK = 32  # tokens per backward chunk (the library's)


def backward_counts(cfg):
    """Work the backward pass must do, with Q the backward chunk, as (first kernel's flops, the
    other's, bytes).  Scalar decay: per group the causal C B^T; per head the causal dY X^T,
    (S o L)^T dY, (L o DYX)^T C and (L o DYX) B ((Q + 1) flops per token and dimension each), and
    the four N x P contractions of the carried state's terms (B^T G, G x, H dy and the update of G)
    in the reverse walk; the recomputed state (B^T X) in the checkpoint pass.  Diagonal decay: the
    local kernel's intra-chunk sums and local sums S, U; the state-terms kernel's three carried
    products.  Bytes: every input and output gradient once."""
    Bsz, T, H, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["ngroups"]
    P, N, Q = cfg["headdim"], cfg["dstate"], BWD_CHUNK
    sx = 4 if cfg["dtype"] == "fp32" else 2
    diag = cfg["decay"] == "diag"
    if diag:
        # per head: the scores with the decay inside (per n), dB, dC and M per (t, s, n), and the
        # local sums S and U: the local kernel's work
        f_walk = Bsz * T * H * ((2 * P + 4 * N) * (Q + 1) + 4 * N * P)
    else:
        f_walk = Bsz * T * (G * N * (Q + 1) + H * ((2 * P + 2 * N) * (Q + 1) + 8 * N * P))
    # the checkpoint pass (scalar); the state-terms kernel's three carried-state products (diagonal)
    f_states = Bsz * T * H * (6 if diag else 2) * N * P
    K = N if diag else 1
    nbytes = Bsz * T * (3 * H * P * sx + 2 * G * N * sx + 2 * G * N * 4 + 2 * 4 * H * K) \
        + (2 * 4 * H if cfg["skip"] else 0) + 4 * Bsz * H * N * P * (2 * int(cfg["init"]) + int(cfg["final"]))
    return f_walk, f_states, nbytes


def run_backward(args, cfg, inp, dev):
    """One JSON line for the backward pass on the workload: tokens/s of ssd_backward, the
    dominant kernel (the reverse walk) against the fp32 matrix peak, and the fp64 adjoint on the
    host's cores for the first batch element."""
    import torch
    import ssd_inputs
    import ssd_chunked_scan_02_amd as ssd
    f_walk, f_states, nbytes = backward_counts(cfg)
    og = ssd_inputs.output_gradients(cfg, ssd_inputs.SEEDS[args.workload] + 1000)
    copies = args.copies or min(32, max(2, math.ceil(1.0e9 / nbytes)))
    bufs = []
    for _ in range(copies):
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
        g["dy"] = og["dy"].to(dev)
        g["dfinal"] = og["dfinal"].to(dev) if cfg["final"] else None
        bufs.append(g)
    dims = ssd.dims_for(bufs[0]["x"], bufs[0]["log_a"], bufs[0]["B"])
    ws = torch.empty(max(1, ssd.ssd_backward_workspace_bytes(dims)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = HipEvents()

    def step(i, events=None):
        g = bufs[i % copies]
        kw = dict(D=g.get("D"), init_state=g.get("init_state"), dfinal=g["dfinal"], want_dD=cfg["skip"],
                  want_dinit=cfg["init"], workspace=ws, stream=stream)
        if events is None:
            return ssd.ssd_backward(g["x"], g["log_a"], g["B"], g["C"], g["dy"], **kw)
        return ssd.ssd_backward_profiled(g["x"], g["log_a"], g["B"], g["C"], g["dy"], events=events, **kw)[1]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    begin, end = ev.create(), ev.create()
    kept = None  # the gradients of the last timed call on the first input copy
    ev.lib.hipEventRecord(begin, stream.cuda_stream)
    for i in range(K):
        r = step(i)
        if i % copies == 0:
            kept = r
    ev.lib.hipEventRecord(end, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(begin, end) / K
    step_events = [[ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)] for _ in range(K)]
    launches = None
    for i in range(K):
        launches = step(i, step_events[i])
    torch.cuda.synchronize()
    per_kernel = [[ev.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in step_events] for k in range(launches)]
    for e in step_events:
        for h in e:
            ev.destroy(h)
    kernel_avg = [sum(v) / len(v) for v in per_kernel]
    N, P = cfg["dstate"], cfg["headdim"]
    sfx = "_diag" if cfg["decay"] == "diag" else ""
    # scalar decay, bf16 inputs, N in {32, 64, 128}, P in {32, 64}: the bf16-MFMA kernels
    bf16_path = not sfx and cfg["dtype"] == "bf16" and N in (32, 64, 128) and P in (32, 64)
    peak = BF16_PEAK_TFLOPS if bf16_path else FP32_PEAK_TFLOPS
    if sfx:
        names = ["bwd_local_diag_kernel<%d,%d>" % (N, P), "bwd_scan_diag_kernel<%d,%d>" % (N, P),
                 "bwd_terms_diag_kernel<%d,%d>" % (N, P)]
    elif bf16_path:
        names = ["zero_kernel", "bwd_states_bf16_kernel<%d,%d>" % (N, P), "bwd_walk_bf16_kernel<%d,%d>" % (N, P)]
    else:
        names = ["zero_kernel", "bwd_states_kernel<%d,%d>" % (N, P), "bwd_walk_kernel<%d,%d>" % (N, P)]
    names += ["bwd_reduce_kernel"] if cfg["skip"] else []
    if len(names) != launches:
        names = ["launch%d" % k for k in range(launches)]
    log("backward ms/step %.4f; per kernel avg ms: %s" % (ms, ", ".join("%s %.4f" % kv for kv in zip(names, kernel_avg))))
    walk = next((k for k, n in enumerate(names) if n.startswith("bwd_walk")), max(range(launches), key=lambda k: kernel_avg[k]))
    f_dom = f_states if names[walk].startswith("bwd_terms_diag") else f_walk
    if args.calibrate_copy_mib:
        calibrate_copy(dev, args.calibrate_copy_mib)
    tokens = cfg["batch"] * cfg["seqlen"]
    achieved = f_dom / (kernel_avg[walk] / 1e3) / 1e12
    result = {
        "metric": "SSD backward tokens/s (gradients of x, log a, B, C, D, init) at B=%d,T=%d,H=%d,P=%d,N=%d"
                  % (cfg["batch"], cfg["seqlen"], cfg["nheads"], P, N),
        "value": tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16_path else "f32",
        "data": "synthetic (seeded; the forward workload's inputs, dL/dy ~ N(0,1) in the input dtype)",
        "config": {"workload": args.workload, "pass": "backward", "batch": cfg["batch"], "seqlen": cfg["seqlen"],
                   "nheads": cfg["nheads"], "ngroups": cfg["ngroups"], "headdim": P, "dstate": N,
                   "input_dtype": cfg["dtype"], "backward_chunk": BWD_CHUNK, "parallelism": "single GPU"},
        "tflops": (f_walk + f_states) / (ms / 1e3) / 1e12,
        "kernels_ms": {n: t for n, t in zip(names, kernel_avg)},
        "roofline": {"kernel": names[walk], "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(args.workload + "_bwd", names[walk]),
                     "algorithmic_flops_per_launch": f_dom, "hbm_gbs_whole_step": nbytes / (ms / 1e3) / 1e9},
    }
    if not args.no_cpu_baseline:
        import oracle.backward
        f = ssd_inputs.to_f64
        one = lambda t: None if t is None else f(t[:1])
        threads = oracle.default_threads() if hasattr(oracle, "default_threads") else 1
        reps, t0 = 0, time.perf_counter()
        while True:
            want = oracle.backward.backward(one(inp["x"]), one(inp["log_a"]), one(inp["B"]), one(inp["C"]),
                                            f(inp.get("D")), one(inp.get("init_state")), one(og["dy"]),
                                            one(og["dfinal"]) if cfg["final"] else None, nthreads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        # (the adjoint runs one (batch, group) pair per thread: the sample has G of them)
        result["cpu_baseline"] = {"value": cfg["seqlen"] * reps / el, "unit": "tokens/s",
                                  "cores": min(threads, cfg["ngroups"]),
                                  "kind": "oracle", "cpu_model": cpu_model(),
                                  "sample": "batch element 0 of the workload (%d tokens x %d heads), %d run(s) in "
                                            "%.1f s, fp64 adjoint of the recurrence, OpenMP over (batch, group)"
                                            % (cfg["seqlen"], cfg["nheads"], reps, el)}
        result["parity"] = backward_parity(cfg, kept, want)
    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        sys.exit(1)


def run_varlen(args, cfg, dev):
    """One JSON line for ssd_forward_varlen: the workload's tokens split into args.varlen
    sequences of a seeded log-normal length mix, packed on one token axis; tokens/s of the whole
    packed forward, the dominant kernel against HBM, and the oracle's per-sequence recurrence on
    the host's cores."""
    import torch
    import ssd_inputs
    import ssd_chunked_scan_02_amd as ssd
    seed = ssd_inputs.SEEDS[args.workload]
    total = cfg["batch"] * cfg["seqlen"]
    lengths = ssd_inputs.packed_lengths(args.varlen, total, seed)
    p = ssd_inputs.packed_inputs(cfg, lengths, seed)
    nseq, maxT = len(lengths), p["max_seqlen"]
    H, N, P = cfg["nheads"], cfg["dstate"], cfg["headdim"]
    flops, nbytes, per_token = algorithmic_counts(cfg)
    states = 4 * H * N * P * (int(cfg["init"]) + int(cfg["final"]))
    nbytes += (nseq - cfg["batch"]) * states
    copies = args.copies or min(64, max(2, math.ceil(1.0e9 / nbytes)))
    log("workload %s packed into %d sequences (lengths %d..%d, max %d): %.1f MB algorithmic per step, %d copies"
        % (args.workload, nseq, min(lengths), max(lengths), maxT, nbytes / 1e6, copies))
    cu = p["cu_seqlens"].to(dev)
    bufs = []
    for _ in range(copies):
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in p.items()}
        g["y"] = torch.empty_like(g["x"])
        g["final"] = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev) if cfg["final"] else None
        bufs.append(g)
    dims = ssd.varlen_dims(bufs[0]["x"], bufs[0]["log_a"], bufs[0]["B"], nseq, maxT)
    ws = torch.empty(max(1, ssd.ssd_forward_varlen_workspace_bytes(dims, cfg["chunk"])), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = HipEvents()

    def step(i, events=None):
        g = bufs[i % copies]
        return ssd.ssd_forward_varlen(g["x"], g["log_a"], g["B"], g["C"], cu, maxT, g.get("D"), chunk=cfg["chunk"],
                                      init_state=g.get("init_state"), y=g["y"], final_state=g["final"], workspace=ws,
                                      stream=stream, events=events)[2]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    begin, end = ev.create(), ev.create()
    ev.lib.hipEventRecord(begin, stream.cuda_stream)
    for i in range(K):
        step(i)
    ev.lib.hipEventRecord(end, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(begin, end) / K
    step_events = [[ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)] for _ in range(K)]
    launches = None
    for i in range(K):
        launches = step(i, step_events[i])
    torch.cuda.synchronize()
    per_kernel = [[ev.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in step_events] for k in range(launches)]
    for e in step_events:
        for h in e:
            ev.destroy(h)
    kernel_avg = [sum(v) / len(v) for v in per_kernel]
    names = kernel_names(dict(cfg, seqlen=maxT), segmented=False, packed=nseq, tokens=total)
    if len(names) != launches:
        names = ["launch%d" % k for k in range(launches)]
    dom = max(range(launches), key=lambda k: kernel_avg[k])
    log("varlen ms/step %.4f; per kernel avg ms: %s" % (ms, ", ".join("%s %.4f" % kv for kv in zip(names, kernel_avg))))
    if args.calibrate_copy_mib:
        calibrate_copy(dev, args.calibrate_copy_mib)
    if names[dom].startswith("walk_fast_kernel"):
        dom_bytes = total * (H * P * 4 + 4 * H) + (4 * H if cfg["skip"] else 0) + nseq * states
    else:
        dom_bytes = nbytes
    achieved = dom_bytes / (kernel_avg[dom] / 1e3) / 1e9
    result = {
        "metric": "SSD forward tokens/s, packed variable-length batch (ssd_forward_varlen)",
        "value": total / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded; the workload's value distributions on one packed token axis, lengths log-normal)",
        "config": {"workload": args.workload, "varlen_sequences": nseq, "tokens": total, "max_seqlen": maxT,
                   "min_seqlen": min(lengths), "nheads": H, "ngroups": cfg["ngroups"], "headdim": P, "dstate": N,
                   "chunk": cfg["chunk"], "decay": cfg["decay"], "parallelism": "single GPU"},
        "kernels_ms": {n: t for n, t in zip(names, kernel_avg)},
        "roofline": {"kernel": names[dom], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("%s_varlen%d" % (args.workload, nseq), names[dom]),
                     "algorithmic_bytes_per_launch": dom_bytes, "tokens_per_launch": total},
    }
    if not args.no_cpu_baseline:
        import oracle
        import oracle.varlen
        f = ssd_inputs.to_f64
        a = [f(p["x"]), f(p["log_a"]), f(p["B"]), f(p["C"])]
        threads = oracle.default_threads()
        reps, t0 = 0, time.perf_counter()
        while True:
            ref = oracle.varlen.forward_varlen(oracle.default_oracle(), *a, p["cu_seqlens"].numpy(), f(p.get("D")),
                                               f(p.get("init_state")), want_final=cfg["final"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        result["cpu_baseline"] = {"value": total * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "cpu_model": cpu_model(),
                                  "sample": "the whole packed batch (%d tokens in %d sequences x %d heads), %d run(s) "
                                            "in %.1f s, fp64 recurrence per sequence, OpenMP over heads"
                                            % (total, nseq, H, reps, el)}
        # the timed run's outputs (first input copy) against the oracle's, as one batch element
        yr, fr = ref
        result["parity"] = output_parity(cfg, {"x": p["x"][None], "D": p.get("D")}, bufs[0]["y"][None],
                                         bufs[0]["final"], (yr[None], fr))
    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2_layer")
    ap.add_argument("--backward", action="store_true",
                    help="time ssd_backward (the gradients) instead of the forward pass")
    ap.add_argument("--front-end", choices=("log_a", "dt"), default="log_a",
                    help="decay input: log a (ssd_forward), or dt and A_log (ssd_forward_dt)")
    ap.add_argument("--varlen", type=int, default=0,
                    help="time ssd_forward_varlen: the workload's tokens packed as this many sequences")
    ap.add_argument("--copies", type=int, default=0, help="input copies cycled (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import ssd_inputs
    import ssd_chunked_scan_02_amd as ssd

    cfg = ssd_inputs.config(args.workload)
    seed = ssd_inputs.SEEDS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = ssd_inputs.make_inputs(cfg, seed)
    if args.backward:
        return run_backward(args, cfg, inp, dev)
    if args.varlen:
        return run_varlen(args, cfg, dev)
    fe = args.front_end
    flops, nbytes, per_token = algorithmic_counts(cfg, fe)
    copies = args.copies or min(64, max(2, math.ceil(1.0e9 / nbytes)))
    log("workload %s seed %d: %.2f GFLOP, %.1f MB algorithmic per step, %d copies"
        % (args.workload, seed, flops / 1e9, nbytes / 1e6, copies))

    bufs = []
    for _ in range(copies):
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
        g["y"] = torch.empty_like(g["x"])
        g["final"] = (torch.empty((cfg["batch"], cfg["nheads"], cfg["dstate"], cfg["headdim"]),
                                  dtype=torch.float32, device=dev) if cfg["final"] else None)
        bufs.append(g)
    dims = ssd.dims_for(bufs[0]["x"], bufs[0]["log_a"], bufs[0]["B"])
    ws_need = (ssd.ssd_forward_dt_workspace_bytes(dims, cfg["chunk"], True) if fe == "dt"
               else ssd.ssd_forward_workspace_bytes(dims, cfg["chunk"]))
    ws = torch.empty(max(1, ws_need), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = HipEvents()

    def step(i, events=None):
        g = bufs[i % copies]
        kw = dict(chunk=cfg["chunk"], init_state=g.get("init_state"), y=g["y"],
                  final_state=g["final"], workspace=ws, stream=stream)
        if fe == "dt":
            if events is None:
                ssd.ssd_forward_dt(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"), **kw)
                return None
            return ssd.ssd_forward_dt_profiled(g["x"], g["dt"], g["A_log"], g["B"], g["C"], g.get("D"),
                                               events=events, **kw)[2]
        if events is None:
            ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), **kw)
            return None
        return ssd.ssd_forward_profiled(g["x"], g["log_a"], g["B"], g["C"], g.get("D"),
                                        events=events, **kw)[2]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Throughput: K plain forwards back to back, bracketed by two events on the launch stream.
    K = args.steps
    begin, end = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.lib.hipEventRecord(begin, stream.cuda_stream)
    for i in range(K):
        step(i)
    ev.lib.hipEventRecord(end, stream.cuda_stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(begin, end)
    # Kernel run times: K more forwards whose launches each stamp their own start/end events.
    # Timestamped dispatches cost the queue a few microseconds each, so this pass is kept out
    # of the throughput figure above.
    step_events = [[ev.create() for _ in range(2 * ssd.SSD_MAX_LAUNCHES)] for _ in range(K)]
    t0, t1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.lib.hipEventRecord(t0, stream.cuda_stream)
    launches = None
    for i in range(K):
        launches = step(i, step_events[i])
    ev.lib.hipEventRecord(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    timed_ms = ev.elapsed_ms(t0, t1) / K
    per_kernel = [[ev.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in step_events] for k in range(launches)]
    for e in step_events:
        for h in e:
            ev.destroy(h)

    ms = total_ms / K
    kernel_avg = [sum(v) / len(v) for v in per_kernel]
    dom = max(range(launches), key=lambda k: kernel_avg[k])
    names = kernel_names(cfg, fe)
    if len(names) != launches:
        names = ["launch%d" % k for k in range(launches)]
    log("ms/step %.4f (%.4f with per-launch timing); per kernel avg ms: %s"
        % (ms, timed_ms, ", ".join("%s %.4f" % (n, t) for n, t in zip(names, kernel_avg))))

    if args.calibrate_copy_mib:
        calibrate_copy(dev, args.calibrate_copy_mib)
    copy_gbs = measured_copy_gbs(dev, ev, stream)

    tokens = cfg["batch"] * cfg["seqlen"]
    tok_s = tokens / (ms / 1e3)
    tflops = flops / (ms / 1e3) / 1e12
    peak_tf = FP32_PEAK_TFLOPS if cfg["dtype"] == "fp32" else BF16_PEAK_TFLOPS
    dom_ms = kernel_avg[dom]
    dom_bytes = kernel_bytes(cfg, names[dom], nbytes)
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    profile_key = args.workload if fe == "log_a" else args.workload + "_dt"
    traffic = measured_traffic(profile_key, names[dom])
    result = {
        "metric": "SSD forward tokens/s + TFLOP/s (% MFMA peak) at " + shape_text(cfg),
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else "f32",
        "data": ("synthetic (seeded; x~N(0,1), B,C~N(0,1/N), log a=-softplus(dt)exp(A_log))" if fe == "log_a" else
                 "synthetic (seeded; x~N(0,1), B,C~N(0,1/N), dt and A_log in, log a and the input scale "
                 "softplus(dt) formed in the kernels)"),
        "config": {"workload": args.workload, "batch": cfg["batch"], "seqlen": cfg["seqlen"],
                   "nheads": cfg["nheads"], "ngroups": cfg["ngroups"], "headdim": cfg["headdim"],
                   "dstate": cfg["dstate"], "chunk": cfg["chunk"], "decay": cfg["decay"],
                   "front_end": fe, "parallelism": "single GPU"},
        "tflops": tflops,
        "mfma_peak_frac": tflops / peak_tf,
        "hbm_gbs_whole_step": nbytes / (ms / 1e3) / 1e9,
        "kernels_ms": {n: t for n, t in zip(names, kernel_avg)},
        "dominant_kernel_ms_median_min": [statistics.median(per_kernel[dom]), min(per_kernel[dom])],
        "ms_per_step_with_kernel_timing": timed_ms,
        "roofline": {"kernel": names[dom], "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes,
                     "bytes_per_token": dom_bytes / tokens, "tokens_per_launch": tokens,
                     "forward_bytes_per_token": per_token,
                     "peak_measured_copy": copy_gbs, "frac_of_measured_copy": achieved / copy_gbs},
        "provenance": provenance(args.workload, seed),
    }
    if cfg.get("decode_steps", 0) > 0:
        result["decode"] = time_decode(ssd, cfg, bufs[0], stream, ev, dev)
    ok = True
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle (>= %.0f s)..." % args.cpu_seconds)
        result["cpu_baseline"], ref = cpu_baseline(inp, cfg, args.cpu_seconds, fe)
        # the same oracle run checks the timed kernels' outputs (every copy holds the same inputs)
        result["parity"] = output_parity(cfg, inp, bufs[0]["y"], bufs[0]["final"], ref)
        log("parity: relL2 y %.3e, SSD part %.3e%s -> %s"
            % (result["parity"]["rel_l2_y"], result["parity"]["rel_l2_ssd_part"],
               (", final %.3e" % result["parity"]["rel_l2_final"]) if "rel_l2_final" in result["parity"] else "",
               "ok" if result["parity"]["pass"] else "FAILED"))
        ok = result["parity"]["pass"]
    print(json.dumps(result), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
