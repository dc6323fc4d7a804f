"""GPU parity of dense grouped-query attention (K / V with fewer heads than Q)
against the oracle's grouped-query reference (the dense definition with every
K / V head repeated over its group; dK / dV summed over the group)."""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs
import scaled_dot_product_bwd_amd as sdb
from gpu_helpers import MASK_CODE, TOL, rel_err

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Sq, Sk, H, Hkv, D, dtype):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *shape: torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)
    return mk(B, Sq, H, D), mk(B, Sk, Hkv, D), mk(B, Sk, Hkv, D), mk(B, Sq, H, D)


CASES = [
    # (seed, B, Sq, Sk, H, Hkv, D, dtype, mask, window, causal_flag)
    (201, 2, 256, 256, 8, 2, 128, torch.bfloat16, "causal", 0, False),
    (202, 1, 300, 300, 6, 3, 64, torch.float32, "window", 40, False),
    (203, 2, 100, 250, 4, 1, 64, torch.float32, "keypad", 0, True),
    (204, 1, 160, 96, 8, 4, 32, torch.bfloat16, "none", 0, False),
    (205, 1, 130, 200, 4, 2, 128, torch.float32, "bias", 0, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}-{c[8]}-g{c[4] // c[5]}")
def test_gqa_parity(case):
    seed, B, Sq, Sk, H, Hkv, D, dtype, mask, window, causal = case
    q, k, v, dy = _inputs(seed, B, Sq, Sk, H, Hkv, D, dtype)
    m = None
    if mask == "keypad":
        m = (torch.arange(Sk)[None, :] < torch.tensor([[Sk - 37], [Sk]])).float().view(B, 1, 1, Sk)
    elif mask == "bias":
        m = torch.randn(B, H, Sq, Sk, generator=torch.Generator().manual_seed(seed + 1))
    print(f"[gqa] seed={seed} q={tuple(q.shape)} kv={tuple(k.shape)} {dtype} {mask}", flush=True)
    dev = torch.device("cuda:0")
    dq, dk, dv = sdb.attn_bwd(*(x.to(dev) for x in (q, k, v, dy)), mask_kind=mask, window=window,
                              causal=causal, mask=None if m is None else m.to(dev))
    torch.cuda.synchronize()
    ref = oracle.attn_bwd_gqa(q, k, v, dy, mask_kind=MASK_CODE[mask], window=window,
                              causal_flag=causal, mask=None if m is None else m.double().numpy())
    assert dk.shape == k.shape and dv.shape == v.shape
    scale0 = float(np.max(np.abs(ref["dv"])))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        g64 = got.double().cpu().numpy()
        assert not np.isnan(g64).any()
        e = rel_err(g64, ref[name], scale0)
        assert e <= TOL[dtype], f"{name}: rel err {e:.3e}"


def test_gqa_with_equal_heads_is_mha_bitwise():
    """Hkv = H takes the same path as plain multi-head attention: identical bits."""
    q, k, v, dy = _inputs(206, 2, 192, 192, 4, 4, 64, torch.bfloat16)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    a = sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal")
    args = sdb.make_args(qd, kd, vd, gd, *[torch.empty_like(x) for x in (qd, kd, vd)],
                         mask_kind="causal",
                         workspace=torch.empty(sdb.workspace_bytes(2, 4, 192), dtype=torch.uint8,
                                               device=dev))
    args.Hkv = 0  # "same as H"
    b = [torch.empty_like(x) for x in (qd, kd, vd)]
    args.dq, args.dk, args.dv = (t.data_ptr() for t in b)
    sdb.attn_bwd_stage("all", args)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
