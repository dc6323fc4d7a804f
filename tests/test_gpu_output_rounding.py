"""Bit-exact check of the bf16 output rounding (fp32 accumulator -> bf16 store,
round to nearest, ties to even), in the dense and the paged dK / dV kernels.

Inputs are built so that every fp32 accumulation is exact: Q = 0 makes every
score 0, and each query row sees exactly one key (dense: an additive bias of
-1e30 hides the others; paged: supplied statistics m = 0, l = 1), so P = 1
exactly and dV of a key is a plain sum of bf16 values of dY.  The addends of
each output element (tests/bf16_rounding.py) sum to a bf16 halfway point, a
little above or below one, or three quarters of an ulp, at several exponents
and both signs; the expected bits are the round-to-nearest-even of the exact
rational sum.  dK = dS^T Q is exactly 0 here.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import scaled_dot_product_bwd_amd as sdb
from bf16_rounding import bf16_bits, halfway_columns, rne_bf16

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _bits(t):
    return t.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF


def test_dense_dv_store_rounds_to_nearest_even():
    Sk, D, rows_per_key = 64, 128, 4
    Sq = Sk * rows_per_key
    cols = halfway_columns(Sk * D)
    dy = torch.zeros(1, Sq, 1, D, dtype=torch.float64)
    want = np.zeros((Sk, D), dtype=np.int64)
    for j in range(Sk):
        for d in range(D):
            addends, x = cols[j * D + d]
            for r, a in enumerate(addends):
                dy[0, rows_per_key * j + r, 0, d] = float(a)
            want[j, d] = bf16_bits(rne_bf16(x))
    g = torch.Generator().manual_seed(3)
    k = (0.5 * torch.randn(1, Sk, 1, D, generator=g, dtype=torch.float64)).to(BF)
    v = torch.randn(1, Sk, 1, D, generator=g, dtype=torch.float64).to(BF)
    q = torch.zeros(1, Sq, 1, D, dtype=BF)
    dy = dy.to(BF)
    assert torch.equal(dy.double(), dy.double().to(BF).double())  # addends are bf16 values
    bias = torch.full((1, 1, Sq, Sk), -1e30)
    i = torch.arange(Sq)
    bias[0, 0, i, i // rows_per_key] = 0.0
    dev = torch.device("cuda:0")
    qd, kd, vd, gd, bd = (x.to(dev) for x in (q, k, v, dy, bias))
    outs = tuple(torch.full_like(x, float("nan")) for x in (qd, kd, vd))
    dq, dk, dv = sdb.attn_bwd(qd, kd, vd, gd, mask_kind="bias", mask=bd, out=outs)
    torch.cuda.synchronize()
    got = _bits(dv[0, :, 0, :])
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} dV elements differ from round-to-nearest-even; first "
                           f"(key, d) = {tuple(bad[0])}: got {hex(got[tuple(bad[0])])}, "
                           f"want {hex(want[tuple(bad[0])])}")
    assert torch.all(dk == 0)
    # dQ = dS K with dS = P (dP - delta) scale, zero in exact arithmetic: only
    # rounding of dP - delta is left, tiny against the gradients' scale.
    assert float(dq.float().abs().max()) <= 2e-2 * float(dv.float().abs().max())


def test_paged_dv_store_rounds_to_nearest_even():
    D, heads, kvh, ps = 128, 2, 1, 16
    cols = halfway_columns(D)
    plan = sdb.paged_plan(np.array([16]), np.array([[1]]), np.array([0, 0]), np.array([15, 15]),
                          heads=heads, kv_heads=kvh, page_size=ps, pool_pages=2)
    dy = torch.zeros(2, heads, D, dtype=torch.float64)
    want = np.zeros(D, dtype=np.int64)
    for d in range(D):
        addends, x = cols[d]
        for n, a in enumerate(addends):  # (row, head) = (n // 2, n % 2)
            dy[n // 2, n % 2, d] = float(a)
        want[d] = bf16_bits(rne_bf16(x))
    g = torch.Generator().manual_seed(4)
    k_pool = torch.randn(2 * ps, kvh, D, generator=g, dtype=torch.float64).to(BF)
    v_pool = torch.randn(2 * ps, kvh, D, generator=g, dtype=torch.float64).to(BF)
    q = torch.zeros(2, heads, D, dtype=BF)
    stats = torch.zeros(2, heads, 3)
    stats[..., 1] = 1.0  # m = 0, l = 1: P = exp(0 - 0) / 1 = 1 for every visible token
    dev = torch.device("cuda:0")
    sentinel = torch.full((2 * ps, kvh, D), 0x7FC1, dtype=torch.int16).view(BF)
    dk, dv = sentinel.clone().to(dev), sentinel.clone().to(dev)
    sdb.attn_bwd_paged(q.to(dev), dy.to(BF).to(dev), k_pool.to(dev), v_pool.to(dev),
                       stats.to(dev), plan.to(dev), dk_pool=dk, dv_pool=dv)
    torch.cuda.synchronize()
    got = _bits(dv[ps:, 0, :])
    for t in range(ps):  # every token of the listed page gets the same sum
        assert np.array_equal(got[t], want), (t, np.argwhere(got[t] != want)[:4].tolist())
    assert np.all(_bits(dv[:ps]) == 0x7FC1) and np.all(_bits(dk[:ps]) == 0x7FC1)  # page 0 unlisted
    assert torch.all(dk[ps:] == 0)
