"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same host values, and compare.

The parity metric (per output tensor): max|gpu - ref| / max|ref|, at most 1e-4
for float32 inputs and 2e-2 for bfloat16 inputs.  Where the reference tensor is
identically zero (closed forms such as a single visible key, where dS = 0
exactly), the ratio is undefined; the denominator is then max(1, max|dV_ref|),
the problem's gradient scale, so rounding noise of the GPU's dP - delta is
judged against the size of the gradients it would perturb.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import scaled_dot_product_bwd_amd as sdb

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
MASK_CODE = {"none": 0, "causal": 1, "keypad": 2, "window": 3, "bias": 4}


def rel_err(gpu, ref, zero_ref_scale=1.0) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if not r.size:
        return 0.0
    den = float(np.max(np.abs(r)))
    if den == 0.0:
        den = max(1.0, zero_ref_scale)
    return float(np.max(np.abs(g - r))) / den


def gpu_run(q, k, v, dy, *, wrt="all", mask_kind="none", causal=False, window=0, mask=None,
            threshold=0.5, scale=None, prefill_nan=True, workspace=None):
    """Inputs are CPU tensors; returns CPU float64 numpy results and the stats.
    workspace: None (the binding's choice), "min" (attn_bwd_workspace_bytes:
    never the split form) or "split" (attn_bwd_split_workspace_bytes)."""
    dev = torch.device("cuda:0")
    ws_in = None
    if workspace is not None:
        B_, Sq_, H_, D_ = q.shape
        n = (sdb.workspace_bytes(B_, H_, Sq_) if workspace == "min"
             else sdb.split_workspace_bytes(B_, H_, Sq_, k.shape[1], D_))
        ws_in = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    md = mask.to(dev) if mask is not None else None
    outs = []
    for want, ref in (("q", qd), ("k", kd), ("v", vd)):
        if wrt in ("all", want):
            o = torch.empty_like(ref)
            if prefill_nan:
                o.fill_(float("nan"))
            outs.append(o)
        else:
            outs.append(None)
    (dq, dk, dv), ws = sdb.attn_bwd(qd, kd, vd, gd, wrt=wrt, mask_kind=mask_kind, causal=causal,
                                    window=window, mask=md, threshold=threshold, scale=scale,
                                    out=tuple(outs), return_workspace=True, workspace=ws_in)
    torch.cuda.synchronize()
    B, Sq, H, _ = q.shape
    m, l, d = sdb.row_stats_views(ws, B, H, Sq)
    res = {}
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        res[name] = None if t is None else t.detach().float().cpu().double().numpy()
    res["m"], res["l"], res["delta"] = (x.cpu().double().numpy() for x in (m, l, d))
    return res


def oracle_run(q, k, v, dy, *, mask_kind="none", causal=False, window=0, mask=None,
               threshold=0.5, scale=None, nthreads=None):
    return oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_CODE[mask_kind], causal_flag=causal,
                           window=window, mask=None if mask is None else mask.double().numpy(),
                           threshold=threshold, scale=scale, nthreads=nthreads)


def assert_parity(res, ref, dtype, names=("dq", "dk", "dv"), stats=True, label=""):
    tol = TOL[dtype]
    report = {}
    for n in names:
        if res.get(n) is None:
            continue
        assert not np.isnan(res[n]).any(), f"{label} {n}: NaN left in the output"
        e = rel_err(res[n], ref[n], float(np.max(np.abs(ref["dv"]), initial=0.0)))
        report[n] = e
        assert e <= tol, f"{label} {n}: rel err {e:.3e} > {tol:g}"
    if stats:
        fin = np.isfinite(ref["m"])
        assert np.array_equal(np.isfinite(res["m"]), fin), f"{label} empty-row pattern differs"
        assert np.all(res["l"][~fin] == 0) and np.all(res["delta"][~fin] == 0)
        for n, t in (("m", 1e-5), ("l", 1e-4), ("delta", tol)):
            e = rel_err(res[n][fin], ref[n][fin]) if fin.any() else 0.0
            report[n] = e
            assert e <= t, f"{label} stat {n}: rel err {e:.3e} > {t:g}"
    return report


def sample_heads(x, pairs):
    """[B, S, H, D] -> [1, S, len(pairs), D] holding the (b, h) heads listed."""
    return torch.stack([x[b, :, h, :] for b, h in pairs], dim=1).unsqueeze(0)
