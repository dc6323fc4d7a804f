"""GPU tests of the fused query-major pass (row statistics and dQ together,
attn_bwd_stats_dq; bf16), which attn_bwd uses for bf16 inputs.

dQ comes out as scale (A - delta B) / l with A = sum p~ dP K and B = sum p~ K
accumulated against a lazily moved reference max; these tests check it
against the oracle where that reference moves at every chunk (scores rising
steeply with the key index), on rows dominated by one key (where A - delta B
cancels), under every mask kind, and that the stage calls reproduce
attn_bwd's bits.
"""
import numpy as np
import pytest
import torch

import sdpa_inputs
import scaled_dot_product_bwd_amd as sdb
from gpu_helpers import assert_parity, gpu_run, oracle_run

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


# (S, D): a short case over ragged chunks, and the benchmark's sequence length
# and head width, where a row's statistics move over 32 chunks of 64 keys.
SIZES = [(320, 64), (2048, 128)]


@pytest.mark.parametrize("S,D", SIZES)
@pytest.mark.parametrize("causal", [False, True])
def test_reference_max_moves_every_chunk(causal, S, D):
    """A bias rising 0.4 per key lifts a row's max by ~18 log2 units per 32-key
    chunk, so the reference moves (and A, B, l are rescaled) at every chunk."""
    B, H = 1, 2
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=11, dtype=BF)
    bias = (0.4 * torch.arange(S, dtype=torch.float32)).expand(B, H, S, S).contiguous()
    res = gpu_run(q, k, v, dy, mask_kind="bias", mask=bias, causal=causal)
    ref = oracle_run(q, k, v, dy, mask_kind="bias", mask=bias, causal=causal, nthreads=2)
    print(causal, S, assert_parity(res, ref, BF, label=f"rising bias causal={causal} S={S}"))


@pytest.mark.parametrize("S,D", SIZES)
@pytest.mark.parametrize("qscale", [4.0, 8.0])
def test_peaked_rows(qscale, S, D):
    """Large |q|: most rows are dominated by one key (dP ~ delta there), where
    A - delta B cancels; dQ must stay as accurate as the three-pass path."""
    B, H = 1, 2
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=5, dtype=torch.float64)
    q, k, v, dy = ((qscale * q).to(BF), k.to(BF), v.to(BF), dy.to(BF))
    for mask in ("none", "causal"):
        res = gpu_run(q, k, v, dy, mask_kind=mask)
        ref = oracle_run(q, k, v, dy, mask_kind=mask, nthreads=2)
        print(qscale, S, mask, assert_parity(res, ref, BF, label=f"peaked x{qscale} {mask} S={S}"))


@pytest.mark.parametrize("Sk", [40, 64, 100, 192, 256, 300, 384])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_chunk_counts(mask, Sk):
    """Row blocks over one to six 64-key chunks.  Each chunk's phase C runs in
    the next chunk's step, so this covers a block's first chunk (nothing
    pending), the rotation of four K buffers, and the last chunk's phase C
    after the loop, with the first chunk masked (window, ragged key end) or
    not (no mask, causal with the query rows at the end of the keys)."""
    B, H, Sq, D = 1, 2, 200, 64
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=300 + Sk, dtype=BF)
    window = 70 if mask == "window" else 0
    res = gpu_run(q, k, v, dy, mask_kind=mask, window=window)
    ref = oracle_run(q, k, v, dy, mask_kind=mask, window=window, nthreads=2)
    print(mask, Sk, assert_parity(res, ref, BF, label=f"{mask} Sk={Sk}"))


@pytest.mark.parametrize("mask,window", [("window", 40), ("keypad", 0), ("bias", 0)])
def test_masks_bf16(mask, window):
    B, H, Sq, Sk, D = 2, 2, 150, 290, 128
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=123, dtype=BF)
    m = None
    if mask == "keypad":
        m = torch.ones(B, 1, 1, Sk)
        m[0, ..., 200:] = 0.0
        m[1, ..., :17] = 0.0
    elif mask == "bias":
        g = torch.Generator().manual_seed(9)
        m = torch.randn(B, H, Sq, Sk, generator=g, dtype=torch.float64).float()
    res = gpu_run(q, k, v, dy, mask_kind=mask, window=window, mask=m, causal=mask != "window")
    ref = oracle_run(q, k, v, dy, mask_kind=mask, window=window, mask=m, causal=mask != "window")
    print(mask, assert_parity(res, ref, BF, label=mask))


@pytest.mark.parametrize("D", [32, 64, 128])
def test_stage_calls_equal_attn_bwd_bitwise(D):
    """attn_bwd_stats_dq then attn_bwd_kv on one stream gives attn_bwd's bits;
    attn_bwd_row_stats (32-key chunks) gives the same statistics up to rounding."""
    B, S, H = 2, 333, 3
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=40 + D, dtype=BF)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    res = []
    for stages in (("all",), ("stats_dq", "kv"), ("row_stats",)):
        outs = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
        w = torch.full((sdb.workspace_bytes(B, H, S),), 0xFF, dtype=torch.uint8, device=dev)
        a = sdb.make_args(qd, kd, vd, gd, *outs, mask_kind="causal", workspace=w)
        for st in stages:
            sdb.attn_bwd_stage(st, a)
        res.append((outs, w))
    torch.cuda.synchronize()
    for x, y in zip(res[0][0], res[1][0]):
        assert torch.equal(x, y)
    assert torch.equal(res[0][1], res[1][1])
    m0, l0, d0 = sdb.row_stats_views(res[0][1], B, H, S)
    m1, l1, d1 = sdb.row_stats_views(res[2][1], B, H, S)
    assert torch.equal(m0, m1)  # the max is exact
    assert torch.allclose(l0, l1, rtol=1e-5, atol=0) and torch.allclose(d0, d1, rtol=1e-4, atol=1e-5)


def test_dq_only_and_stats_only_calls():
    """wrt=K runs the fused pass without its dQ store: dQ memory is untouched."""
    B, S, H, D = 1, 200, 2, 64
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=3, dtype=BF)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    dq = torch.full_like(qd, 7.0)
    dk, dv = torch.empty_like(kd), torch.empty_like(vd)
    w = torch.empty(sdb.workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
    a = sdb.make_args(qd, kd, vd, gd, dq, dk, dv, mask_kind="causal", workspace=w, wrt="k")
    sdb.attn_bwd_stage("all", a)
    torch.cuda.synchronize()
    assert torch.all(dq == 7.0)
    ref = oracle_run(q, k, v, dy, mask_kind="causal")
    full = gpu_run(q, k, v, dy, mask_kind="causal")
    assert np.array_equal(dk.float().cpu().double().numpy(), full["dk"])
    assert_parity(full, ref, BF)
