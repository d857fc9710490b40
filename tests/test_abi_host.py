"""The C ABI on a machine without a GPU: the library loads, exports every function that
include/ssd.h declares, sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import ssd_chunked_scan_02_amd as ssd
from ssd_chunked_scan_02_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.library_path()):
        from ssd_chunked_scan_02_amd.build import build
        build()
    return ssd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["ssd_backward", "ssd_backward_dt", "ssd_backward_dt_varlen",
                                    "ssd_backward_dt_varlen_workspace_bytes", "ssd_backward_dt_workspace_bytes",
                                    "ssd_backward_profiled", "ssd_backward_varlen",
                                    "ssd_backward_varlen_workspace_bytes", "ssd_backward_workspace_bytes",
                                    "ssd_forward", "ssd_forward_dt", "ssd_forward_dt_profiled",
                                    "ssd_forward_dt_varlen", "ssd_forward_dt_varlen_workspace_bytes",
                                    "ssd_forward_dt_workspace_bytes", "ssd_forward_noalloc", "ssd_forward_profiled",
                                    "ssd_forward_varlen", "ssd_forward_varlen_workspace_bytes",
                                    "ssd_forward_workspace_bytes", "ssd_noalloc_scratch_bytes", "ssd_step",
                                    "ssd_step_dt", "ssd_strerror"]


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert ssd.ssd_strerror(code)
    assert "unknown" in ssd.ssd_strerror(7)


def mamba2_dims(**kw):
    d = dict(batch=8, seqlen=2048, nheads=24, ngroups=1, headdim=64, dstate=128, dtype=1, decay=0)
    d.update(kw)
    return Dims(**d)


def n_pairs(nt):
    m = nt // 2
    return m * (m + 1) if nt % 2 == 0 else (m + 1) * (m + 1)


def test_workspace_bytes(lib):
    # bf16, scalar decay, head dim 64, N in {64,128}, chunk in {64,128}: per (batch, group,
    # chunk) the bf16 score-tile pairs (1 KiB each) and the B^T and C^T operands (N * chunk * 2
    # bytes each), plus log a head-major over whole chunks (4 bytes per (batch, head, padded token))
    fast = lambda batch, heads, groups, nch, N, Q: (batch * groups * nch * (n_pairs(Q // 16) * 1024 + N * Q * 4)
                                                    + batch * heads * nch * Q * 4)
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(), 128) == fast(8, 24, 1, 16, 128, 128)
    # ragged: 2050 tokens -> 17 chunks
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(seqlen=2050), 128) == fast(8, 24, 1, 17, 128, 128)
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(ngroups=8, nheads=64), 64) == fast(8, 64, 8, 32, 128, 64)
    # chunk 256 runs as 128-token chunks; with few (batch, head) units on a long sequence the
    # walk is split into segments (here 32 units, 512 chunks -> 8 segments of 64 chunks: one
    # walk workgroup per CU), which adds an fp32 state and a log2 decay per (segment, unit), the
    # decays padded to 256 bytes
    seg = 8 * 32 * (128 * 64 * 4) + (8 * 32 * 4 + 255) // 256 * 256
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(batch=1, nheads=32, seqlen=65536), 256) == \
        fast(1, 32, 1, 512, 128, 128) + seg
    # other shapes: causal 16x16 fp32 score tiles per (batch, group, chunk)
    tiles = lambda nblk, Q: nblk * (Q // 16) * (Q // 16 + 1) // 2 * 1024
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(dtype=0), 64) == tiles(8 * 32, 64)
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(headdim=32), 256) == tiles(8 * 8, 256)
    # diagonal decay needs no workspace unless its walk is segmented: then per (segment, unit) an
    # fp32 local state, an fp32 start state and a log2 decay per state row (2 units, 64 chunks ->
    # 16 segments)
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(decay=1, dstate=64), 64) == 0
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(decay=1, dstate=64, batch=1, nheads=2, seqlen=4096), 64) == \
        2 * 16 * 2 * 64 * 64 * 4 + (16 * 2 * 64 * 4 + 255) // 256 * 256
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(seqlen=0), 128) == 0
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(), 48) == 0        # unsupported chunk
    assert ssd.ssd_forward_workspace_bytes(mamba2_dims(nheads=5, ngroups=2), 64) == 0


def test_fast_path_limits(lib):
    """Shapes whose in-chunk byte offsets would not fit in 32 bits, or with more heads per group
    than the prep kernel moves, leave the bf16 fast path for the generic one (whose workspace is
    the fp32 score tiles alone)."""
    tiles = lambda nblk, Q: nblk * (Q // 16) * (Q // 16 + 1) // 2 * 1024
    # 8 heads per group, d_state 128: one token of x and B, C spans (64 + 128 / 8) * 2 = 160
    # bytes per head, so a 128-token chunk passes 2^31 bytes from 104858 heads on
    for nheads, fast in ((104864, False), (104848, True)):
        d = mamba2_dims(batch=1, seqlen=128, nheads=nheads, ngroups=nheads // 8)
        assert (ssd.ssd_forward_workspace_bytes(d, 128) != tiles(nheads // 8, 128)) == fast
    # the prep kernel moves log a for at most 64 heads per group at 128-token chunks
    for nheads, fast in ((65, False), (64, True)):
        d = mamba2_dims(batch=1, seqlen=128, nheads=nheads, ngroups=1)
        assert (ssd.ssd_forward_workspace_bytes(d, 128) != tiles(1, 128)) == fast


def test_diag_shapes_supported_and_not(lib):
    d = mamba2_dims(decay=1, dstate=64)
    assert call_forward(lib, d, chunk=128) == ssd.SSD_ERR_UNSUPPORTED      # diag chunk <= 64
    assert call_forward(lib, mamba2_dims(decay=1, dstate=256), chunk=64) == ssd.SSD_ERR_UNSUPPORTED


FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced: validation fails first


def call_forward(lib, dims, chunk=128, ptrs=None, ws_bytes=1 << 30, **over):
    p = dict(x=FAKE, log_a=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE, final=None, ws=FAKE)
    p.update(ptrs or {})
    p.update(over)
    return lib.ssd_forward(ctypes.byref(dims), p["x"], p["log_a"], p["B"], p["C"], p["D"], chunk,
                           p["init"], p["y"], p["final"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("field,value", [("batch", -1), ("seqlen", -5), ("nheads", 0),
                                         ("ngroups", 0), ("headdim", 0), ("dstate", -2),
                                         ("dtype", 7), ("decay", 3)])
def test_forward_rejects_bad_dims(lib, field, value):
    assert call_forward(lib, mamba2_dims(**{field: value})) == ssd.SSD_ERR_INVALID


def test_forward_rejects_groups_not_dividing_heads(lib):
    assert call_forward(lib, mamba2_dims(nheads=6, ngroups=4)) == ssd.SSD_ERR_INVALID


@pytest.mark.parametrize("chunk", [0, 8, 48, 100, 512])
def test_forward_rejects_unsupported_chunk(lib, chunk):
    assert call_forward(lib, mamba2_dims(), chunk=chunk) == ssd.SSD_ERR_UNSUPPORTED


@pytest.mark.parametrize("over", [dict(dstate=48), dict(headdim=96), dict(dstate=512),
                                  dict(dstate=256, headdim=128), dict(dstate=16)])
def test_forward_rejects_unsupported_shapes(lib, over):
    assert call_forward(lib, mamba2_dims(**over)) == ssd.SSD_ERR_UNSUPPORTED


def test_fp32_shapes_that_exceed_lds_are_unsupported(lib):
    assert call_forward(lib, mamba2_dims(dtype=0), chunk=256) == ssd.SSD_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["x", "log_a", "B", "C", "y"])
def test_forward_rejects_null_required_pointer(lib, name):
    assert call_forward(lib, mamba2_dims(), **{name: None}) == ssd.SSD_ERR_INVALID


@pytest.mark.parametrize("name", ["x", "log_a", "B", "C", "D", "init", "y", "final", "ws"])
def test_forward_rejects_misaligned_pointer(lib, name):
    assert call_forward(lib, mamba2_dims(), **{name: FAKE + 4}) == ssd.SSD_ERR_ALIGN


def test_forward_rejects_small_workspace(lib):
    need = ssd.ssd_forward_workspace_bytes(mamba2_dims(), 128)
    assert call_forward(lib, mamba2_dims(), ws_bytes=need - 1) == ssd.SSD_ERR_INVALID
    assert call_forward(lib, mamba2_dims(), ws=None) == ssd.SSD_ERR_INVALID


def test_empty_batch_is_a_no_op(lib):
    # nothing to do: returns success without touching the (fake) pointers or the GPU
    assert call_forward(lib, mamba2_dims(batch=0), ptrs=dict(x=None, log_a=None, B=None, C=None,
                                                             y=None, ws=None), ws_bytes=0) == 0


def call_step(lib, dims, **over):
    p = dict(state=FAKE, x=FAKE, la=FAKE, B=FAKE, C=FAKE, D=None, y=FAKE)
    p.update(over)
    return lib.ssd_step(ctypes.byref(dims), p["state"], p["x"], p["la"], p["B"], p["C"], p["D"],
                        p["y"], None)


def test_step_rejects_bad_arguments(lib):
    d = mamba2_dims(batch=4, nheads=64, ngroups=8)
    assert call_step(lib, mamba2_dims(nheads=0)) == ssd.SSD_ERR_INVALID
    assert call_step(lib, d, state=None) == ssd.SSD_ERR_INVALID
    assert call_step(lib, d, y=None) == ssd.SSD_ERR_INVALID
    assert call_step(lib, d, x=FAKE + 2) == ssd.SSD_ERR_ALIGN
    assert call_step(lib, mamba2_dims(dstate=48)) == ssd.SSD_ERR_UNSUPPORTED


def test_profiled_forward_rejects_short_event_array(lib):
    d = mamba2_dims()
    events = (ctypes.c_void_p * 7)(*([None] * 7))  # one short of 2 * SSD_MAX_LAUNCHES
    n = ctypes.c_int(-1)
    rc = lib.ssd_forward_profiled(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 128, None, FAKE,
                                  None, FAKE, 1 << 30, None, events, 7, ctypes.byref(n))
    assert rc == ssd.SSD_ERR_INVALID and n.value == 0


# ---- the discretisation front-end (ssd_forward_dt, ssd_step_dt)
def test_dt_workspace_bytes(lib):
    # fused bf16 scalar path: ssd_forward's workspace, plus log2 of the input scale head-major
    # (4 bytes per (batch, head, padded token)) when the input is scaled
    d = mamba2_dims()
    plain = ssd.ssd_forward_workspace_bytes(d, 128)
    assert ssd.ssd_forward_dt_workspace_bytes(d, 128, False) == plain
    assert ssd.ssd_forward_dt_workspace_bytes(d, 128, True) == plain + 8 * 24 * 16 * 128 * 4
    # fused diagonal walk: the same as ssd_forward
    dd = mamba2_dims(decay=1, dstate=64, batch=1, nheads=2, seqlen=4096)
    assert ssd.ssd_forward_dt_workspace_bytes(dd, 64, True) == ssd.ssd_forward_workspace_bytes(dd, 64)
    # generic composition: the walk's own workspace, log a, and (scaled) the scaled input, each
    # part on a 256-byte boundary
    up = lambda v: (v + 255) // 256 * 256
    g = mamba2_dims(dtype=0, batch=2, seqlen=300, nheads=3, dstate=64)
    own = ssd.ssd_forward_workspace_bytes(g, 64)
    la = 2 * 300 * 3 * 4
    assert ssd.ssd_forward_dt_workspace_bytes(g, 64, False) == up(up(own) + la)
    assert ssd.ssd_forward_dt_workspace_bytes(g, 64, True) == up(up(own) + la) + 2 * 300 * 3 * 64 * 4
    gd = mamba2_dims(decay=1, dtype=0, batch=1, seqlen=100, nheads=2, dstate=16, headdim=32)
    assert ssd.ssd_forward_dt_workspace_bytes(gd, 32, True) == up(1 * 100 * 2 * 16 * 4) + 100 * 2 * 32 * 4
    assert ssd.ssd_forward_dt_workspace_bytes(mamba2_dims(seqlen=0), 128, True) == 0
    assert ssd.ssd_forward_dt_workspace_bytes(mamba2_dims(), 48, True) == 0


def call_forward_dt(lib, dims, chunk=128, ws_bytes=1 << 30, **over):
    p = dict(x=FAKE, dt=FAKE, dt_bias=None, A_log=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE, final=None,
             ws=FAKE)
    p.update(over)
    return lib.ssd_forward_dt(ctypes.byref(dims), p["x"], p["dt"], p["dt_bias"], p["A_log"], 1, p["B"], p["C"],
                              p["D"], chunk, p["init"], p["y"], p["final"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "dt", "A_log", "B", "C", "y"])
def test_forward_dt_rejects_null_required_pointer(lib, name):
    assert call_forward_dt(lib, mamba2_dims(), **{name: None}) == ssd.SSD_ERR_INVALID


@pytest.mark.parametrize("name", ["dt", "dt_bias", "A_log"])
def test_forward_dt_rejects_misaligned_pointer(lib, name):
    assert call_forward_dt(lib, mamba2_dims(), **{name: FAKE + 4}) == ssd.SSD_ERR_ALIGN


def test_forward_dt_rejects_small_workspace_and_bad_shapes(lib):
    need = ssd.ssd_forward_dt_workspace_bytes(mamba2_dims(), 128, True)
    assert call_forward_dt(lib, mamba2_dims(), ws_bytes=need - 1) == ssd.SSD_ERR_INVALID
    assert call_forward_dt(lib, mamba2_dims(), chunk=48) == ssd.SSD_ERR_UNSUPPORTED
    assert call_forward_dt(lib, mamba2_dims(nheads=6, ngroups=4)) == ssd.SSD_ERR_INVALID
    assert call_forward_dt(lib, mamba2_dims(batch=0), x=None, dt=None, A_log=None, B=None, C=None, y=None,
                           ws=None, ws_bytes=0) == 0


def test_step_dt_rejects_bad_arguments(lib):
    def call(dims, **over):
        p = dict(state=FAKE, x=FAKE, dt=FAKE, bias=None, A_log=FAKE, B=FAKE, C=FAKE, D=None, y=FAKE)
        p.update(over)
        return lib.ssd_step_dt(ctypes.byref(dims), p["state"], p["x"], p["dt"], p["bias"], p["A_log"], 1, p["B"],
                               p["C"], p["D"], p["y"], None)
    d = mamba2_dims(batch=4, nheads=64, ngroups=8)
    assert call(d, dt=None) == ssd.SSD_ERR_INVALID
    assert call(d, A_log=None) == ssd.SSD_ERR_INVALID
    assert call(d, bias=FAKE + 8) == ssd.SSD_ERR_ALIGN
    assert call(mamba2_dims(dstate=48)) == ssd.SSD_ERR_UNSUPPORTED


# ---- the backward pass
def test_backward_workspace_bytes(lib):
    # one fp32 N x P state per (batch, head, 32 tokens), then 4 bytes per (batch, head), each part
    # on a 256-byte boundary
    up = lambda v: (v + 255) // 256 * 256
    d = mamba2_dims(batch=2, seqlen=300, nheads=4)
    assert ssd.ssd_backward_workspace_bytes(d) == up(2 * 4 * 10 * 128 * 64 * 4) + up(2 * 4 * 4)
    assert ssd.ssd_backward_workspace_bytes(mamba2_dims(batch=0)) == 0
    assert ssd.ssd_backward_workspace_bytes(mamba2_dims(decay=1)) == 0          # diagonal decay: N <= 64
    # diagonal decay: the dD sums per (batch, head, chunk); a gradient slot per checkpoint; an fp32
    # decay per (batch, head, chunk, state dim); the intra-chunk terms per (b, t, h) row, fp32: dx [P],
    # dB, dC, dcum [N] each
    dd = mamba2_dims(decay=1, dstate=64, batch=1, seqlen=100, nheads=2)
    rows = 1 * 100 * 2
    assert ssd.ssd_backward_workspace_bytes(dd) == 2 * up(1 * 2 * 4 * 64 * 64 * 4) + up(1 * 2 * 4 * 4) + \
        up(1 * 2 * 4 * 64 * 4) + up(rows * 64 * 4) + 3 * up(rows * 64 * 4)
    assert ssd.ssd_backward_workspace_bytes(mamba2_dims(headdim=128)) == 0      # P <= 64


def call_backward(lib, dims, ws_bytes=1 << 30, **over):
    p = dict(x=FAKE, la=FAKE, B=FAKE, C=FAKE, D=None, init=None, dy=FAKE, dfin=None, dx=FAKE, dla=FAKE, dB=FAKE,
             dC=FAKE, dD=None, dinit=None, ws=FAKE)
    p.update(over)
    return lib.ssd_backward(ctypes.byref(dims), p["x"], p["la"], p["B"], p["C"], p["D"], p["init"], p["dy"],
                            p["dfin"], p["dx"], p["dla"], p["dB"], p["dC"], p["dD"], p["dinit"], p["ws"], ws_bytes,
                            None)


@pytest.mark.parametrize("name", ["x", "la", "B", "C", "dy", "dx", "dla", "dB", "dC"])
def test_backward_rejects_null_required_pointer(lib, name):
    assert call_backward(lib, mamba2_dims(), **{name: None}) == ssd.SSD_ERR_INVALID


def test_backward_rejects_bad_arguments(lib):
    assert call_backward(lib, mamba2_dims(), dD=FAKE + 4) == ssd.SSD_ERR_ALIGN
    assert call_backward(lib, mamba2_dims(decay=1)) == ssd.SSD_ERR_UNSUPPORTED
    assert call_backward(lib, mamba2_dims(dstate=256)) == ssd.SSD_ERR_UNSUPPORTED
    need = ssd.ssd_backward_workspace_bytes(mamba2_dims())
    assert call_backward(lib, mamba2_dims(), ws_bytes=need - 1) == ssd.SSD_ERR_INVALID


def test_backward_dt_workspace_bytes(lib):
    # the front-end's rows (log a, dx_in, dlog a and the dA_log terms: K = 1 scalar, N diagonal, per
    # row; the scaled input with scale_input; dD terms), each on a 256-byte boundary, then the
    # backward pass's own workspace
    up = lambda v: (v + 255) // 256 * 256
    fn = lib.ssd_backward_dt_workspace_bytes
    for decay, N, P in ((0, 128, 64), (1, 64, 32)):
        d = mamba2_dims(batch=2, seqlen=300, nheads=4, decay=decay, dstate=N, headdim=P)
        rows, K = 2 * 300 * 4, (N if decay else 1)
        inner = ssd.ssd_backward_workspace_bytes(d)
        own = up(rows * K * 4) + up(rows * P * 2) + up(rows * K * 4) + up(rows * K * 4) + up(rows * 4)
        assert fn(ctypes.byref(d), 0) == own + inner
        assert fn(ctypes.byref(d), 1) == own + up(rows * P * 2) + inner
    assert fn(ctypes.byref(mamba2_dims(decay=1)), 1) == 0                  # diagonal decay: N <= 64
    assert fn(ctypes.byref(mamba2_dims(batch=0)), 1) == 0


# ---- packed variable-length batches
def call_varlen(lib, dims, cu=FAKE, total=1000, ws_bytes=1 << 30, **over):
    p = dict(x=FAKE, la=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE, fin=None, ws=FAKE)
    p.update(over)
    return lib.ssd_forward_varlen(ctypes.byref(dims), cu, total, p["x"], p["la"], p["B"], p["C"], p["D"], 64,
                                  p["init"], p["y"], p["fin"], p["ws"], ws_bytes, None, None, 0, None)


def packed_as_one_bytes(H, G, N, cap, Q=128, P=64):
    """The fast path's workspace for a packed batch walked as one sequence of up to `cap` tokens:
    the batched layout of one sequence of cap tokens (score pairs, B^T, C^T, log a head-major) with
    segment states for the most segments any length gives (256 // H when 2 H <= 256), then one int
    of token flags per token of whole chunks."""
    up = lambda v: (v + 255) // 256 * 256
    nch = -(-cap // Q)
    blk = G * nch
    own = blk * n_pairs(Q // 16) * 1024 + 2 * blk * N * Q * 2 + H * nch * Q * 4
    segs = 256 // H if 2 * H <= 256 else 1
    if segs > 1:
        own += segs * H * N * P * 4 + up(segs * H * 4)
    return own + nch * Q * 4


def test_varlen_workspace_bytes(lib):
    # the larger of two layouts on the fast path: a [batch][seqlen] batch's workspace without
    # segmented walks (the same as ssd_forward's when the batched walk is not segmented either,
    # less when it is), with, for at most 4096 sequences, their order by length (4 bytes each);
    # and the packed batch walked as one sequence of batch * seqlen tokens (no per-sequence states)
    many = mamba2_dims(batch=64, seqlen=1000)
    up = lambda v: (v + 255) // 256 * 256
    seq_by_seq = ssd.ssd_forward_workspace_bytes(many, 128) + up(64 * 4)
    as_one = packed_as_one_bytes(24, 1, 128, 64 * 1000)
    assert as_one > seq_by_seq
    assert ssd.ssd_forward_varlen_workspace_bytes(many, 128) == as_one
    lots = mamba2_dims(batch=5000, seqlen=64)
    assert ssd.ssd_forward_varlen_workspace_bytes(lots, 128) == max(ssd.ssd_forward_workspace_bytes(lots, 128),
                                                                     packed_as_one_bytes(24, 1, 128, 5000 * 64))
    few = mamba2_dims(batch=1, seqlen=65536, nheads=32)
    # (one sequence: walked as one it is the batched layout, segmented alike, plus the flags)
    assert ssd.ssd_forward_varlen_workspace_bytes(few, 128) == ssd.ssd_forward_workspace_bytes(few, 128) + 65536 * 4
    assert ssd.ssd_forward_varlen_workspace_bytes(few, 128) == packed_as_one_bytes(32, 1, 128, 65536)
    dd = mamba2_dims(decay=1, dstate=64, batch=1, nheads=2, seqlen=4096)
    assert ssd.ssd_forward_varlen_workspace_bytes(dd, 64) == 0 < ssd.ssd_forward_workspace_bytes(dd, 64)
    assert ssd.ssd_forward_varlen_workspace_bytes(mamba2_dims(), 48) == 0


def test_varlen_rejects_bad_arguments(lib):
    d = mamba2_dims(batch=4, seqlen=512)
    assert call_varlen(lib, d, total=-1) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, d, cu=None) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, d, cu=FAKE + 4) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, d, x=None) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, d, y=FAKE + 2) == ssd.SSD_ERR_ALIGN
    need = ssd.ssd_forward_varlen_workspace_bytes(d, 64)
    assert call_varlen(lib, d, ws_bytes=need - 1) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, mamba2_dims(dstate=48)) == ssd.SSD_ERR_UNSUPPORTED
    # nothing to do: no sequences, or no tokens and no final state wanted (no HIP call)
    assert call_varlen(lib, mamba2_dims(batch=0), cu=None, total=0) == ssd.SSD_OK
    assert call_varlen(lib, d, total=0, x=None, la=None, B=None, C=None, y=None) == ssd.SSD_OK


def test_dt_varlen_workspace_and_checks(lib):
    # the fused paths: the packed log a form's workspace (plus log2 of the input scale on the scalar
    # fast path); the generic composition adds rows for batch * seqlen tokens
    d = mamba2_dims(batch=4, seqlen=512)
    assert ssd.ssd_forward_dt_varlen_workspace_bytes(d, 128, False) == ssd.ssd_forward_varlen_workspace_bytes(d, 128)
    assert ssd.ssd_forward_dt_varlen_workspace_bytes(d, 128, True) == \
        ssd.ssd_forward_varlen_workspace_bytes(d, 128) + 4 * 24 * 4 * 128 * 4
    g = mamba2_dims(batch=2, seqlen=300, nheads=3, dtype=0, dstate=16)
    assert ssd.ssd_forward_dt_varlen_workspace_bytes(g, 64, True) == ssd.ssd_forward_dt_workspace_bytes(g, 64, True)
    fn = lib.ssd_forward_dt_varlen
    args = lambda dims, total: (ctypes.byref(dims), FAKE, total, FAKE, FAKE, None, FAKE, 1, FAKE, FAKE, None, 128,
                                None, FAKE, None, FAKE, 1 << 30, None, None, 0, None)
    assert fn(*args(d, 4 * 512 + 1)) == ssd.SSD_ERR_INVALID        # more tokens than batch * seqlen
    assert fn(*args(d, -1)) == ssd.SSD_ERR_INVALID
    assert call_varlen(lib, d, total=4 * 512 + 1) == ssd.SSD_ERR_INVALID


def test_backward_varlen_checks(lib):
    d = mamba2_dims(batch=4, seqlen=512)
    assert ssd.ssd_forward_varlen_workspace_bytes  # (the forward's query is separate)
    assert lib.ssd_backward_varlen_workspace_bytes(ctypes.byref(d)) == ssd.ssd_backward_workspace_bytes(d)
    fn = lib.ssd_backward_varlen
    def call(dims, cu=FAKE, total=1000, ws=FAKE, ws_bytes=1 << 32, **over):
        p = dict(x=FAKE, la=FAKE, B=FAKE, C=FAKE, dy=FAKE, dx=FAKE, dla=FAKE, dB=FAKE, dC=FAKE)
        p.update(over)
        return fn(ctypes.byref(dims), cu, total, p["x"], p["la"], p["B"], p["C"], None, None, p["dy"], None, p["dx"],
                  p["dla"], p["dB"], p["dC"], None, None, ws, ws_bytes, None, None, 0, None)
    assert call(d, total=4 * 512 + 1) == ssd.SSD_ERR_INVALID
    assert call(d, total=-1) == ssd.SSD_ERR_INVALID
    assert call(d, cu=None) == ssd.SSD_ERR_INVALID
    assert call(d, cu=FAKE + 4) == ssd.SSD_ERR_INVALID
    assert call(d, dy=None) == ssd.SSD_ERR_INVALID
    assert call(d, ws_bytes=ssd.ssd_backward_workspace_bytes(d) - 1) == ssd.SSD_ERR_INVALID
    assert call(mamba2_dims(decay=1)) == ssd.SSD_ERR_UNSUPPORTED


def test_noalloc_rejects_before_any_hip_call(lib):
    """ssd_forward_noalloc: a workload whose workspace exceeds the fixed scratch array fails with
    SSD_ERR_SCRATCH, and bad arguments with the codes of ssd_forward, all before any HIP call (so
    also on a machine without a GPU)."""
    cap = lib.ssd_noalloc_scratch_bytes()
    assert cap == 96 << 20
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every check fails first
    big = Dims(batch=4, seqlen=8192, nheads=64, ngroups=8, headdim=64, dstate=128, dtype=1, decay=0)
    assert lib.ssd_forward_workspace_bytes(ctypes.byref(big), 128) > cap
    args = (fake, fake, fake, fake, None, 128, None, fake, None, None)
    assert lib.ssd_forward_noalloc(ctypes.byref(big), *args) == ssd.SSD_ERR_SCRATCH
    fits = mamba2_dims()
    assert 0 < lib.ssd_forward_workspace_bytes(ctypes.byref(fits), 128) <= cap
    # a null input, a misaligned output, an unsupported chunk
    assert lib.ssd_forward_noalloc(ctypes.byref(fits), None, fake, fake, fake, None, 128, None, fake, None,
                                   None) == ssd.SSD_ERR_INVALID
    assert lib.ssd_forward_noalloc(ctypes.byref(fits), fake, fake, fake, fake, None, 128, None,
                                   ctypes.c_void_p((1 << 20) + 8), None, None) == ssd.SSD_ERR_ALIGN
    assert lib.ssd_forward_noalloc(ctypes.byref(fits), *((fake,) * 4), None, 48, None, fake, None,
                                   None) == ssd.SSD_ERR_UNSUPPORTED
