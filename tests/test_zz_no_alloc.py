"""ssd_forward_noalloc on the GPU, called through the C ABI: its outputs equal ssd_forward's on the
same inputs bit for bit (the same kernels, with the workspace in the library's fixed per-GPU
scratch array), on calls in a row whose inputs shrink (each call finds the previous call's records
in the array), on the fast, segmented, diagonal and generic paths, and the results stay within the
oracle's bounds.  A workload larger than the array is rejected before any launch."""
import ctypes

import pytest
import torch

import ssd_chunked_scan_02_amd as ssd
import ssd_inputs
from gpu_helpers import announce, compare, oracle_forward, to_gpu

pytestmark = pytest.mark.gpu


def _noalloc(lib, g, chunk, y, fin):
    dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.ssd_forward_noalloc(ctypes.byref(dims), p(g["x"]), p(g["log_a"]), p(g["B"]), p(g["C"]), p(g.get("D")),
                                   int(chunk), p(g.get("init_state")), p(y), p(fin), stream)


# each sequence: a larger call, then smaller ones (the array keeps the previous call's records)
SEQUENCES = [
    [("mamba2_layer", dict()),                                                    # the whole layer shape
     ("mamba2_layer", dict(batch=4, seqlen=1000, nheads=8, init=True)),
     ("mamba2_layer", dict(batch=1, seqlen=300, nheads=3))],
    [("long_seq", dict()),                                                        # 58 MiB of workspace
     ("long_seq", dict(seqlen=20000, nheads=4))],
    [("mamba2_layer", dict(batch=1, seqlen=3001, nheads=2, init=True)),          # segmented walk
     ("mamba2_layer", dict(batch=1, seqlen=1500, nheads=2, init=True))],
    [("diag_multiscale", dict(batch=2, seqlen=2001, nheads=2, init=True)),       # segmented diagonal walk
     ("diag_multiscale", dict(batch=1, seqlen=300, nheads=3))],
    [("tiny_fp32", dict(seqlen=400, skip=True, init=True, nheads=2)),             # generic fp32 walk
     ("tiny_fp32", dict(seqlen=130))],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["fast", "long-seq", "segmented", "diag", "generic-fp32"])
def test_noalloc_matches_forward(seq):
    lib = ssd.load_library()
    for i, (name, over) in enumerate(seq):
        cfg = ssd_inputs.config(name, **over)
        announce("noalloc call %d: %s %s" % (i, name, over))
        inp = ssd_inputs.make_inputs(cfg, 301 + i)
        g = to_gpu(inp)
        dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
        assert ssd.ssd_forward_workspace_bytes(dims, cfg["chunk"]) <= lib.ssd_noalloc_scratch_bytes()
        y0, f0 = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), chunk=cfg["chunk"],
                                 init_state=g.get("init_state"), final_state=True)
        y = torch.full_like(y0, float("nan"))
        fin = torch.full_like(f0, float("nan"))
        rc = _noalloc(lib, g, cfg["chunk"], y, fin)
        assert rc == ssd.SSD_OK, ssd.ssd_strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                           y0.view(torch.int16) if y0.dtype == torch.bfloat16 else y0)
        assert torch.equal(fin, f0)
        compare(inp, y, fin, oracle_forward(inp), cfg["dtype"], True, "noalloc call %d %s" % (i, name))


def test_noalloc_rejects_a_workload_larger_than_its_array():
    lib = ssd.load_library()
    cfg = ssd_inputs.config("gqa_decode", decode_steps=0)  # 183 MiB of workspace
    g = to_gpu(ssd_inputs.make_inputs(cfg, 307))
    dims = ssd.dims_for(g["x"], g["log_a"], g["B"])
    assert ssd.ssd_forward_workspace_bytes(dims, cfg["chunk"]) > lib.ssd_noalloc_scratch_bytes()
    y = torch.empty_like(g["x"])
    announce("noalloc oversized")
    assert _noalloc(lib, g, cfg["chunk"], y, None) == ssd.SSD_ERR_SCRATCH
