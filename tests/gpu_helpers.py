"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and
the fp64 oracle on the same stored inputs, and compare them by relative L2 error."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ssd_inputs
import ssd_chunked_scan_02_amd as ssd

# relative L2 error bounds: fp32 inputs, bf16 inputs (accumulation in fp32 in both)
TOL = {"fp32": 1e-5, "bf16": 2e-2}
# unit roundoff of the output dtype: y is rounded once (to nearest even) after the skip term
# is added, so the SSD part y - D x inherits an error of up to this times |y| per element
OUT_ROUNDOFF = {"fp32": 2.0 ** -24, "bf16": 2.0 ** -8}


def announce(msg: str):
    print("[gpu case] " + msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = float(np.linalg.norm(want.ravel()))
    num = float(np.linalg.norm((got - want).ravel()))
    return num / den if den > 0 else num


def to_gpu(inp: dict) -> dict:
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}


def gpu_forward(g: dict, chunk: int, want_final: bool):
    y, fin = ssd.ssd_forward(g["x"], g["log_a"], g["B"], g["C"], g.get("D"), chunk=chunk,
                             init_state=g.get("init_state"), final_state=bool(want_final))
    torch.cuda.synchronize()
    return y, fin


def oracle_forward(inp: dict, units=None):
    """fp64 oracle on the stored inputs; ``units`` = list of (b, h) to evaluate (each head is
    independent), or None for all.  Returns dict (b, h) -> (y [T,P], final [N,P]).
    Sampled units are gathered into one oracle call (one unit per batch row) so that the
    oracle's threads share them."""
    f = ssd_inputs.to_f64
    nb, T, H, P = inp["x"].shape
    G = inp["B"].shape[2]
    if units is None:
        units = [(b, h) for b in range(nb) for h in range(H)]
    if not units:
        return {}
    bs = torch.tensor([u[0] for u in units])
    hs = torch.tensor([u[1] for u in units])
    gs = hs // (H // G)
    x = f(inp["x"][bs, :, hs].unsqueeze(2))                 # [U, T, 1, P]
    la = f(inp["log_a"][bs, :, hs].unsqueeze(2))            # [U, T, 1] or [U, T, 1, N]
    Bm = f(inp["B"][bs, :, gs].unsqueeze(2))
    Cm = f(inp["C"][bs, :, gs].unsqueeze(2))
    h0 = None if inp.get("init_state") is None else f(inp["init_state"][bs, hs].unsqueeze(1))
    y, fin = oracle.forward(x, la, Bm, Cm, None, h0)
    if inp.get("D") is not None:
        d = f(inp["D"])[hs.numpy()]
        y = y + d[:, None, None, None] * x
    return {u: (y[i, :, 0], fin[i, 0]) for i, u in enumerate(units)}


def compare(inp: dict, y_gpu, fin_gpu, ref: dict, dtype: str, check_final: bool, label: str):
    """relL2 over the evaluated units of y, of the SSD part y - D x, and of the final state."""
    yg = y_gpu.float().cpu().numpy().astype(np.float64)
    x = ssd_inputs.to_f64(inp["x"])
    D = ssd_inputs.to_f64(inp.get("D"))
    keys = sorted(ref)
    got_y = np.stack([yg[b, :, h] for (b, h) in keys])
    want_y = np.stack([ref[k][0] for k in keys])
    skip = np.stack([(D[h] if D is not None else 0.0) * x[b, :, h] for (b, h) in keys])
    e_y = rel_l2(got_y, want_y)
    e_ssd = rel_l2(got_y - skip, want_y - skip)
    tol = TOL[dtype]
    # the SSD part is judged after removing the output rounding it cannot avoid: that rounding
    # is relative to the whole of y, which the skip term may dominate
    ssd_norm = float(np.linalg.norm((want_y - skip).ravel()))
    y_norm = float(np.linalg.norm(want_y.ravel()))
    tol_ssd = tol + (OUT_ROUNDOFF[dtype] * y_norm / ssd_norm if ssd_norm > 0 else 0.0)
    msg = "%s: relL2 y %.3e  ssd-part %.3e (tol %.2e)" % (label, e_y, e_ssd, tol_ssd)
    ok = e_y <= tol and e_ssd <= tol_ssd
    if check_final:
        fg = fin_gpu.cpu().numpy().astype(np.float64)
        e_f = rel_l2(np.stack([fg[b, h] for (b, h) in keys]), np.stack([ref[k][1] for k in keys]))
        msg += "  final %.3e" % e_f
        ok = ok and e_f <= tol
    announce(msg + "  (tol %.0e)" % tol)
    assert np.all(np.isfinite(got_y)), label + ": non-finite outputs"
    assert ok, msg
    return e_y


def per_unit_rel_l2(got, want):
    """relL2 of every (batch, head) unit of [B, T, H, ...] arrays over its own elements
    (units whose reference is all zeros report their absolute error)."""
    d = (np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    w = np.asarray(want, dtype=np.float64)
    axes = tuple(a for a in range(d.ndim) if a not in (0, 2))
    num = np.sqrt((d * d).sum(axis=axes))
    den = np.sqrt((w * w).sum(axis=axes))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def compare_all_units(inp: dict, y_gpu, fin_gpu, dtype: str, label: str):
    """Every (batch, head) unit of a forward against the oracle run over the whole batch: the
    pooled relL2 of y, of the SSD part y - D x and of the final state, and the same per unit
    (an error confined to one unit is not diluted by the others).  The SSD part's bound adds
    the output rounding it cannot avoid, per unit as pooled."""
    f = ssd_inputs.to_f64
    x = f(inp["x"])
    D = f(inp.get("D"))
    want_y, want_f = oracle.forward(x, f(inp["log_a"]), f(inp["B"]), f(inp["C"]), D, f(inp.get("init_state")))
    got_y = y_gpu.double().cpu().numpy()
    got_f = fin_gpu.double().cpu().numpy()
    skip = np.zeros_like(x) if D is None else D[None, None, :, None] * x
    tol, u = TOL[dtype], OUT_ROUNDOFF[dtype]
    e_y, e_f = rel_l2(got_y, want_y), rel_l2(got_f, want_f)
    e_ssd = rel_l2(got_y - skip, want_y - skip)
    y_norm = float(np.linalg.norm(want_y.ravel()))
    ssd_norm = float(np.linalg.norm((want_y - skip).ravel()))
    tol_ssd = tol + (u * y_norm / ssd_norm if ssd_norm > 0 else 0.0)
    uy = per_unit_rel_l2(got_y, want_y)
    ussd = per_unit_rel_l2(got_y - skip, want_y - skip)
    axes = (1, 3)
    uy_norm = np.sqrt((want_y ** 2).sum(axis=axes))
    ussd_norm = np.sqrt(((want_y - skip) ** 2).sum(axis=axes))
    utol_ssd = tol + np.where(ussd_norm > 0, u * uy_norm / np.where(ussd_norm > 0, ussd_norm, 1.0), 0.0)
    # final states per unit: [B, H, N, P] -> relL2 over (N, P)
    df = got_f - want_f
    uf = np.sqrt((df ** 2).sum(axis=(2, 3))) / np.maximum(np.sqrt((want_f ** 2).sum(axis=(2, 3))), 1e-300)
    worst = np.unravel_index(int(np.argmax(uy)), uy.shape)
    announce("%s: relL2 y %.3e ssd-part %.3e (tol %.2e) final %.3e; worst unit %s: y %.3e, max per unit "
             "ssd-part/bound %.3f, final %.3e (tol %.0e)"
             % (label, e_y, e_ssd, tol_ssd, e_f, tuple(int(v) for v in worst), float(uy.max()),
                float((ussd / utol_ssd).max()), float(uf.max()), tol))
    assert np.all(np.isfinite(got_y)) and np.all(np.isfinite(got_f)), label + ": non-finite outputs"
    assert e_y <= tol and e_ssd <= tol_ssd and e_f <= tol, (e_y, e_ssd, e_f)
    assert float(uy.max()) <= tol, "unit %s: y %.3e" % (worst, float(uy.max()))
    assert float((ussd / utol_ssd).max()) <= 1.0, "a unit's SSD part is over its bound"
    assert float(uf.max()) <= tol, "a unit's final state: %.3e" % float(uf.max())
