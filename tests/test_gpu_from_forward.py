"""GPU parity of the dense backward from a forward's saved statistics
(attn_bwd_from_forward: per-row log-sum-exp and the output O) against the
oracle.  The oracle supplies lse = m + log(l) and O = P V from its own float64
forward (O rounded to the input dtype, as a forward would store it)."""
import numpy as np
import pytest
import torch

import sdpa_inputs
import scaled_dot_product_bwd_amd as sdb
from gpu_helpers import TOL, oracle_run, rel_err

pytestmark = pytest.mark.gpu


def _lse(ref):
    with np.errstate(divide="ignore"):
        return np.where(ref["l"] > 0, ref["m"] + np.log(np.where(ref["l"] > 0, ref["l"], 1.0)), -np.inf)


CASES = [
    (2, "causal", 0, False),          # fp32 [2, 512, 8, 64]
    (4, "keypad", 0, True),           # fp32, padding + causal flag, offset 896
    (4, "bias", 0, False),            # fp32, additive bias
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"config{c[0]}-{c[1]}")
def test_from_forward_parity(case):
    k_cfg, mask, window, causal = case
    d = sdpa_inputs.dense_config_inputs(k_cfg)
    q, k, v, dy = d["q"], d["k"], d["v"], d["dy"]
    B, Sk = q.shape[0], k.shape[1]
    m = (d["valid"].reshape(B, 1, 1, Sk) if mask == "keypad" else d["bias"] if mask == "bias"
         else None)
    ref = oracle_run(q, k, v, dy, mask_kind=mask, causal=causal, window=window, mask=m)
    dev = torch.device("cuda:0")
    lse = torch.from_numpy(_lse(ref).astype(np.float32)).to(dev)
    o = torch.from_numpy(ref["out"]).to(q.dtype).to(dev)
    print(f"[fwd] config{k_cfg} {mask} q={tuple(q.shape)} {q.dtype}", flush=True)
    dq, dk, dv = sdb.attn_bwd(*(x.to(dev) for x in (q, k, v, dy)), mask_kind=mask, causal=causal,
                              window=window, mask=None if m is None else m.to(dev),
                              fwd_lse=lse, fwd_out=o)
    torch.cuda.synchronize()
    scale0 = float(np.max(np.abs(ref["dv"])))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = got.double().cpu().numpy()
        assert not np.isnan(g).any()
        e = rel_err(g, ref[name], scale0)
        assert e <= TOL[q.dtype], f"{name}: rel err {e:.3e}"


def test_from_forward_bf16_with_empty_rows():
    """bf16, a batch whose keys are all padded away (every row sees nothing:
    lse = -inf, zero gradients), next to an ordinary batch."""
    g = torch.Generator().manual_seed(301)
    B, S, H, D = 2, 192, 4, 128
    q, k, v, dy = (torch.randn(B, S, H, D, generator=g, dtype=torch.float64).to(torch.bfloat16)
                   for _ in range(4))
    valid = torch.ones(B, 1, 1, S)
    valid[1] = 0.0
    ref = oracle_run(q, k, v, dy, mask_kind="keypad", mask=valid)
    dev = torch.device("cuda:0")
    lse = torch.from_numpy(_lse(ref).astype(np.float32)).to(dev)
    o = torch.from_numpy(ref["out"]).to(torch.bfloat16).to(dev)
    dq, dk, dv = sdb.attn_bwd(*(x.to(dev) for x in (q, k, v, dy)), mask_kind="keypad",
                              mask=valid.to(dev), fwd_lse=lse, fwd_out=o)
    torch.cuda.synchronize()
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        gg = got.double().cpu().numpy()
        assert np.all(gg[1] == 0.0), name
        e = rel_err(gg, ref[name], float(np.max(np.abs(ref["dv"]))))
        assert e <= TOL[torch.bfloat16], f"{name}: rel err {e:.3e}"


def test_from_forward_window_full_size_sampled():
    """The bf16 [4, 2048, 16, 128] window-256 workload from forward statistics,
    checked on two sampled (b, h) heads."""
    d = sdpa_inputs.dense_config_inputs(3)
    q, k, v, dy = d["q"], d["k"], d["v"], d["dy"]
    dev = torch.device("cuda:0")
    heads = [(0, 3), (3, 12)]
    # the oracle's statistics for the sampled heads; the other heads get zeros
    # (finite inputs whose outputs are not compared; heads are independent)
    B, S, H, D = q.shape
    lse = np.zeros((B, H, S))
    O = np.zeros((B, S, H, D))
    refs = {}
    for (b, h) in heads:
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        r = oracle_run(sl(q), sl(k), sl(v), sl(dy), mask_kind="window", window=256)
        lse[b, h] = _lse(r)[0, 0]
        O[b, :, h] = r["out"][0, :, 0]
        refs[(b, h)] = r
    dq, dk, dv = sdb.attn_bwd(*(x.to(dev) for x in (q, k, v, dy)), mask_kind="window", window=256,
                              fwd_lse=torch.from_numpy(lse.astype(np.float32)).to(dev),
                              fwd_out=torch.from_numpy(O).to(torch.bfloat16).to(dev))
    torch.cuda.synchronize()
    for (b, h), r in refs.items():
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = rel_err(got[b, :, h].double().cpu().numpy(), r[name][0, :, 0])
            assert e <= TOL[torch.bfloat16], f"({b},{h}) {name}: rel err {e:.3e}"


@pytest.mark.parametrize("D,dtype", [(64, torch.bfloat16), (128, torch.bfloat16),
                                     (64, torch.float32)])
def test_from_forward_wrt_subsets_bitwise(D, dtype):
    """Every `wrt` takes the same statistics (formed in the dQ kernel's
    prologue), so each gradient equals the wrt=all call's bit for bit; the
    wrt=all call itself is checked against the oracle."""
    B, S, H = 2, 200, 3
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=31, dtype=dtype)
    ref = oracle_run(q, k, v, dy, mask_kind="causal")
    dev = torch.device("cuda:0")
    lse = torch.from_numpy(_lse(ref).astype(np.float32)).to(dev)
    o = torch.from_numpy(ref["out"]).to(q.dtype).to(dev)
    args = [x.to(dev) for x in (q, k, v, dy)]
    print(f"[fwd-wrt] D={D} q={tuple(q.shape)} {dtype}", flush=True)
    full = sdb.attn_bwd(*args, mask_kind="causal", fwd_lse=lse, fwd_out=o)
    torch.cuda.synchronize()
    scale0 = float(np.max(np.abs(ref["dv"])))
    for name, got in zip(("dq", "dk", "dv"), full):
        e = rel_err(got.double().cpu().numpy(), ref[name], scale0)
        assert e <= TOL[dtype], f"{name}: rel err {e:.3e}"
    for i, w in enumerate(("q", "k", "v")):
        one = sdb.attn_bwd(*args, wrt=w, mask_kind="causal", fwd_lse=lse, fwd_out=o)
        torch.cuda.synchronize()
        assert torch.equal(one[i], full[i]), w
