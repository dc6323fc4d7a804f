"""GPU parity of the dense path (C ABI -> HIP kernels) against the CPU oracle.

Workloads follow the five configurations of the build (see sdpa_inputs.py).
Every output element of every named workload is compared with the oracle,
including all 64 (batch, head) heads of the full bf16 [4, 2048, 16, 128] one
(window 256 and plain causal; the oracle runs them on 16 host threads), and
every named workload is run twice: the second run must reproduce the first
bit for bit (no atomics, fixed reduction orders).
"""
import numpy as np
import pytest
import torch

import sdpa_inputs
from gpu_helpers import (TOL, assert_parity, gpu_run, oracle_run, rel_err, sample_heads)

ORACLE_THREADS = 16  # the host share of one GPU on the test machines


def _rerun_bitwise(first, *args, **kw):
    """Runs the same call again and requires identical bits in every output and
    statistic (NaN-free outputs: the first run's parity check rejects NaN)."""
    again = gpu_run(*args, **kw)
    for n in ("dq", "dk", "dv", "m", "l", "delta"):
        if first.get(n) is not None:
            assert np.array_equal(first[n], again[n]), f"{n}: rerun differs"

pytestmark = pytest.mark.gpu


def _cfg_inputs(k):
    d = sdpa_inputs.dense_config_inputs(k)
    return d, d["q"], d["k"], d["v"], d["dy"]


def test_config1_fp32_no_mask():
    d, q, k, v, dy = _cfg_inputs(1)
    res = gpu_run(q, k, v, dy)
    ref = oracle_run(q, k, v, dy)
    print("config1", assert_parity(res, ref, torch.float32, label="config1"))
    _rerun_bitwise(res, q, k, v, dy)


def test_config2_fp32_causal():
    d, q, k, v, dy = _cfg_inputs(2)
    res = gpu_run(q, k, v, dy, mask_kind="causal")
    ref = oracle_run(q, k, v, dy, mask_kind="causal")
    print("config2", assert_parity(res, ref, torch.float32, label="config2"))
    _rerun_bitwise(res, q, k, v, dy, mask_kind="causal")


@pytest.mark.parametrize("case", ["keypad", "keypad_causal", "bias", "bias_causal"])
def test_config4_fp32_padding_and_bias(case):
    d, q, k, v, dy = _cfg_inputs(4)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    causal = case.endswith("causal")
    if case.startswith("keypad"):
        mask, kind = d["valid"].reshape(B, 1, 1, Sk), "keypad"
    else:
        mask, kind = d["bias"], "bias"
    res = gpu_run(q, k, v, dy, mask_kind=kind, causal=causal, mask=mask)
    ref = oracle_run(q, k, v, dy, mask_kind=kind, causal=causal, mask=mask)
    print("config4", case, assert_parity(res, ref, torch.float32, label=case))
    _rerun_bitwise(res, q, k, v, dy, mask_kind=kind, causal=causal, mask=mask)


# The split form of the fp32 query-major passes (key pieces merged in order),
# which a workspace of attn_bwd_split_workspace_bytes enables where the
# (query block, head) workgroups would leave most of the GPU idle, against the
# one-workgroup-per-block form and the oracle: configs 2 and 4, and a ragged
# case (Sq not a multiple of the block, Sk not of the chunk, causal pieces that
# see nothing).  Grouped-query shapes take the split form in test_gpu_gqa.py.
SPLIT_CASES = {
    "config2_causal": dict(cfg=2, kind="causal", causal=False),
    "config4_keypad_causal": dict(cfg=4, kind="keypad", causal=True),
    "config4_bias": dict(cfg=4, kind="bias", causal=False),
    "ragged_causal": dict(cfg=None, kind="causal", causal=False),
    "few_keys_many_queries": dict(cfg="fk", kind="causal", causal=False),
}


def _split_inputs(c):
    if c["cfg"] is None:
        q, k, v, dy, _ = sdpa_inputs.dense_inputs(1, 200, 1000, 4, 32, seed=77)
        return q, k, v, dy, None
    if c["cfg"] == "fk":  # 2 key blocks per head against 2000 queries: the dK / dV pass splits
        q, k, v, dy, _ = sdpa_inputs.dense_inputs(1, 2000, 250, 2, 64, seed=79)
        return q, k, v, dy, None
    d, q, k, v, dy = _cfg_inputs(c["cfg"])
    B, Sk = q.shape[0], k.shape[1]
    mask = None
    if c["kind"] == "keypad":
        mask = d["valid"].reshape(B, 1, 1, Sk)
    elif c["kind"] == "bias":
        mask = d["bias"]
    return q, k, v, dy, mask


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_fp32_split_form_against_oracle_and_direct_form(case):
    c = SPLIT_CASES[case]
    q, k, v, dy, mask = _split_inputs(c)
    kw = dict(mask_kind=c["kind"], causal=c["causal"], mask=mask)
    split = gpu_run(q, k, v, dy, workspace="split", **kw)
    direct = gpu_run(q, k, v, dy, workspace="min", **kw)
    ref = oracle_run(q, k, v, dy, **kw)
    print(case, "split", assert_parity(split, ref, torch.float32, label=case + " split"))
    print(case, "direct", assert_parity(direct, ref, torch.float32, label=case + " direct"))
    _rerun_bitwise(split, q, k, v, dy, workspace="split", **kw)
    # dK / dV read the statistics: the two forms' statistics agree to rounding,
    # so everything stays within the fp32 tolerance of each other too
    for n in ("dq", "dk", "dv"):
        e = rel_err(split[n], direct[n])
        assert e <= TOL[torch.float32], f"{case} {n}: split vs direct {e:.3e}"


BF16_SPLIT_CASES = {
    # few query blocks against many keys: the fused statistics + dQ pass splits
    "causal_offset": dict(B=1, H=4, Sq=256, Sk=4096, D=128, kind="causal", causal=False, window=0),
    "keypad_causal": dict(B=2, H=2, Sq=200, Sk=3000, D=64, kind="keypad", causal=True, window=0),
    "bias": dict(B=1, H=2, Sq=130, Sk=2600, D=32, kind="bias", causal=False, window=0),
    "window": dict(B=1, H=3, Sq=300, Sk=5000, D=128, kind="window", causal=False, window=700),
}


@pytest.mark.parametrize("case", list(BF16_SPLIT_CASES))
def test_bf16_split_form_against_oracle_and_direct_form(case):
    c = BF16_SPLIT_CASES[case]
    q, k, v, dy, g = sdpa_inputs.dense_inputs(c["B"], c["Sq"], c["Sk"], c["H"], c["D"], seed=81,
                                              dtype=torch.bfloat16)
    mask = None
    if c["kind"] == "keypad":
        mask, _ = sdpa_inputs.keypad_valid(g, c["B"], c["Sk"], c["Sk"] // 4)
        mask = mask.reshape(c["B"], 1, 1, c["Sk"])
    elif c["kind"] == "bias":
        mask = sdpa_inputs.bias_normal(g, c["B"], c["H"], c["Sq"], c["Sk"])
    kw = dict(mask_kind=c["kind"], causal=c["causal"], window=c["window"], mask=mask)
    split = gpu_run(q, k, v, dy, workspace="split", **kw)
    direct = gpu_run(q, k, v, dy, workspace="min", **kw)
    ref = oracle_run(q, k, v, dy, **kw)
    print(case, "split", assert_parity(split, ref, torch.bfloat16, label=case + " split"))
    print(case, "direct", assert_parity(direct, ref, torch.bfloat16, label=case + " direct"))
    _rerun_bitwise(split, q, k, v, dy, workspace="split", **kw)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_split_form_fully_masked_rows(dtype):
    """Key padding that hides every key of batch 1 (its rows see nothing: every
    piece's partial is empty, the merge must give m = -inf, l = 0, delta = 0
    and zero dQ rows) and most keys of batch 0 (pieces past the valid keys are
    empty), in the split form, against the oracle."""
    B, H, Sq, Sk, D = 2, 2, 100, 2000, 64
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=82, dtype=dtype)
    valid = torch.ones(B, Sk)
    valid[0, 300:] = 0.0
    valid[1, :] = 0.0
    mask = valid.reshape(B, 1, 1, Sk)
    kw = dict(mask_kind="keypad", mask=mask)
    split = gpu_run(q, k, v, dy, workspace="split", **kw)
    ref = oracle_run(q, k, v, dy, **kw)
    print("fully masked", dtype, assert_parity(split, ref, dtype, label="fully masked split"))
    assert np.all(split["dq"][1] == 0) and np.all(split["dk"][1] == 0) and np.all(split["dv"][1] == 0)
    assert np.all(np.isneginf(split["m"].reshape(B, H, Sq)[1]))


def _random_case(seed):
    """A seeded random dense case: shape, head size, dtype and mask."""
    r = np.random.default_rng(seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 5))
    Sq, Sk = int(r.integers(1, 400)), int(r.integers(1, 3000))
    D = int(r.choice([32, 64, 128]))
    dtype = torch.bfloat16 if r.integers(0, 2) else torch.float32
    kind = str(r.choice(["none", "causal", "window", "keypad", "bias"]))
    return dict(B=B, H=H, Sq=Sq, Sk=Sk, D=D, dtype=dtype, kind=kind,
                window=int(r.integers(0, 600)) if kind == "window" else 0,
                causal=bool(r.integers(0, 2)) if kind in ("keypad", "bias") else False)


@pytest.mark.parametrize("seed", range(900, 912))
def test_random_shapes_with_split_workspace(seed):
    """Seeded random shapes, head sizes, types and masks, each with a
    split-sized workspace (the split forms where the grid is small, the
    one-workgroup-per-block forms elsewhere), against the oracle."""
    c = _random_case(seed)
    print(f"[random] seed {seed}: {c}", flush=True)
    q, k, v, dy, g = sdpa_inputs.dense_inputs(c["B"], c["Sq"], c["Sk"], c["H"], c["D"], seed=seed,
                                              dtype=c["dtype"])
    mask = None
    if c["kind"] == "keypad":
        mask, _ = sdpa_inputs.keypad_valid(g, c["B"], c["Sk"], c["Sk"] // 3)
        mask = mask.reshape(c["B"], 1, 1, c["Sk"])
    elif c["kind"] == "bias":
        mask = sdpa_inputs.bias_normal(g, c["B"], c["H"], c["Sq"], c["Sk"])
    kw = dict(mask_kind=c["kind"], causal=c["causal"], window=c["window"], mask=mask)
    res = gpu_run(q, k, v, dy, workspace="split", **kw)
    ref = oracle_run(q, k, v, dy, nthreads=ORACLE_THREADS, **kw)
    print(seed, assert_parity(res, ref, c["dtype"], label=f"random {seed}"))


def test_bf16_kv_split_through_the_stage_calls():
    """bf16: the fused statistics + dQ pass (never split), then the dK / dV pass
    in split form (64-row query chunks) with a split-sized workspace, against
    the oracle."""
    import scaled_dot_product_bwd_amd as sdb
    dev = torch.device("cuda:0")
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(2, 1500, 200, 2, 128, seed=80, dtype=torch.bfloat16)
    ref = oracle_run(q, k, v, dy, mask_kind="causal")
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    outs = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
    ws = torch.empty(sdb.split_workspace_bytes(2, 2, 1500, 200, 128), dtype=torch.uint8, device=dev)
    a = sdb.make_args(qd, kd, vd, gd, *outs, mask_kind="causal", workspace=ws)
    sdb.attn_bwd_stage("stats_dq", a)
    sdb.attn_bwd_stage("kv", a)
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    sdb.attn_bwd_stage("stats_dq", a)
    sdb.attn_bwd_stage("kv", a)
    torch.cuda.synchronize()
    for n, o, f, r in zip(("dq", "dk", "dv"), outs, first, (ref["dq"], ref["dk"], ref["dv"])):
        g = o.float().cpu().double().numpy()
        assert not np.isnan(g).any(), n
        e = rel_err(g, r, float(np.max(np.abs(ref["dv"]))))
        assert e <= TOL[torch.bfloat16], f"{n}: {e:.3e}"
        assert torch.equal(o.view(torch.int16), f.view(torch.int16)), f"{n}: rerun differs"


def test_split_form_through_the_stage_calls():
    """attn_bwd_row_stats and attn_bwd_dq (bf16 and fp32) with a split-sized
    workspace, against the oracle's statistics and dQ."""
    import scaled_dot_product_bwd_amd as sdb
    dev = torch.device("cuda:0")
    for dtype in (torch.float32, torch.bfloat16):
        q, k, v, dy, _ = sdpa_inputs.dense_inputs(2, 128, 2048, 2, 64, seed=78, dtype=dtype)
        ref = oracle_run(q, k, v, dy, mask_kind="causal")
        qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
        dq = torch.full_like(qd, float("nan"))
        ws = torch.empty(sdb.split_workspace_bytes(2, 2, 128, 2048, 64), dtype=torch.uint8, device=dev)
        a = sdb.make_args(qd, kd, vd, gd, dq, None, None, wrt="q", mask_kind="causal", workspace=ws)
        sdb.attn_bwd_stage("row_stats", a)
        sdb.attn_bwd_stage("dq", a)
        torch.cuda.synchronize()
        m, l, d = (x.cpu().double().numpy() for x in sdb.row_stats_views(ws, 2, 2, 128))
        res = {"dq": dq.float().cpu().double().numpy(), "m": m, "l": l, "delta": d, "dv": None}
        tol = TOL[dtype]
        e = rel_err(res["dq"], ref["dq"])
        assert e <= tol, f"{dtype} stage dq: {e:.3e}"
        for n, t in (("m", 1e-5), ("l", 1e-4), ("delta", tol)):
            e = rel_err(res[n], ref[n])
            assert e <= t, f"{dtype} stage {n}: {e:.3e}"


def _full_size_all_heads(mask_kind, window):
    """The full bf16 [4, 2048, 16, 128] workload: every element of dQ, dK, dV and
    of the statistics against the oracle over all 64 (batch, head) heads, the
    tolerance applied per head as well as over the whole tensor; then a rerun
    that must give the same bits."""
    d, q, k, v, dy = _cfg_inputs(3)
    res = gpu_run(q, k, v, dy, mask_kind=mask_kind, window=window, prefill_nan=True)
    ref = oracle_run(q, k, v, dy, mask_kind=mask_kind, window=window, nthreads=ORACLE_THREADS)
    out = assert_parity(res, ref, torch.bfloat16, label=f"config3 {mask_kind}")
    B, _, H, _ = q.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            for n in ("dq", "dk", "dv"):
                e = rel_err(res[n][b, :, h, :], ref[n][b, :, h, :])
                worst = max(worst, e)
                assert e <= TOL[torch.bfloat16], (n, b, h, e)
    out["worst_head"] = worst
    _rerun_bitwise(res, q, k, v, dy, mask_kind=mask_kind, window=window)
    return out


def test_config3_bf16_window_full_size_all_heads():
    print("config3 window", _full_size_all_heads("window", 256))


def test_config3_bf16_causal_full_size_all_heads():
    """The benchmark's workload: same tensors, plain causal mask."""
    print("config3 causal", _full_size_all_heads("causal", 0))


EDGE = [
    # (B, H, Sq, Sk, D, dtype, mask, window)
    (1, 2, 1, 1, 32, torch.float32, "none", 0),
    (1, 1, 65, 127, 64, torch.float32, "causal", 0),
    (2, 1, 127, 65, 32, torch.float32, "causal", 0),      # Sq > Sk: offset saturates to 0
    (1, 2, 1000, 1000, 128, torch.bfloat16, "causal", 0),
    (1, 1, 300, 333, 128, torch.bfloat16, "window", 64),
    (1, 2, 200, 200, 64, torch.bfloat16, "window", 0),    # each query sees only itself
    (1, 1, 130, 70, 128, torch.float32, "window", 5),     # fully masked rows at the end
    (1, 3, 97, 161, 32, torch.bfloat16, "none", 0),
    (2, 2, 64, 256, 64, torch.bfloat16, "causal", 0),
    (1, 1, 1, 1000, 128, torch.bfloat16, "none", 0),
]


@pytest.mark.parametrize("B,H,Sq,Sk,D,dtype,mask,window", EDGE)
def test_edge_shapes(B, H, Sq, Sk, D, dtype, mask, window):
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=77 + Sq + Sk, dtype=dtype)
    res = gpu_run(q, k, v, dy, mask_kind=mask, window=window)
    ref = oracle_run(q, k, v, dy, mask_kind=mask, window=window)
    print((B, H, Sq, Sk, D, dtype, mask, window), assert_parity(res, ref, dtype))


def test_fully_masked_padding_batch():
    """Key padding that hides every key of batch 1: zero gradients there, zero stats."""
    B, H, Sq, Sk, D = 2, 2, 96, 200, 64
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=5, dtype=torch.float32)
    valid = torch.ones(B, 1, 1, Sk)
    valid[1] = 0.0
    valid[0, ..., 150:] = 0.0
    res = gpu_run(q, k, v, dy, mask_kind="keypad", mask=valid)
    ref = oracle_run(q, k, v, dy, mask_kind="keypad", mask=valid)
    assert_parity(res, ref, torch.float32)
    for n in ("dq", "dk", "dv"):
        assert np.all(res[n][1] == 0.0)
    assert np.all(res["l"][1] == 0) and np.all(np.isneginf(res["m"][1]))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_unseen_keys_get_positive_zero_gradients(dtype):
    """Keys no row sees (hidden by key padding) get dK = dV = +0 exactly, sign
    bit clear: the dK / dV pass accumulates dK negated and stores 0 - scale x."""
    B, H, Sq, Sk, D = 2, 2, 130, 300, 128
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=17, dtype=dtype)
    valid = torch.ones(B, 1, 1, Sk)
    valid[1] = 0.0
    valid[0, ..., 200:] = 0.0
    res = gpu_run(q, k, v, dy, mask_kind="keypad", mask=valid)
    for n in ("dk", "dv"):
        hidden = np.concatenate([res[n][0, 200:].ravel(), res[n][1].ravel()])
        assert np.all(hidden == 0.0), n
        assert not np.signbit(hidden).any(), f"{n}: a negative zero"
    ref = oracle_run(q, k, v, dy, mask_kind="keypad", mask=valid)
    assert_parity(res, ref, dtype)


def test_empty_sequence_dims():
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(1, 0, 40, 2, 32, seed=1, dtype=torch.float32)
    res = gpu_run(q, k, v, dy)
    assert res["dk"].shape == (1, 40, 2, 32) and np.all(res["dk"] == 0) and np.all(res["dv"] == 0)
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(1, 40, 0, 2, 32, seed=1, dtype=torch.float32)
    res = gpu_run(q, k, v, dy)
    assert np.all(res["dq"] == 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wrt_separate_equals_all_bitwise(dtype):
    """rlx-cpu `all_matches_three_separate`: one fused call equals the three
    single-gradient calls; here bit for bit.  The page's hash generator and
    causal mask, with head_dim 32 (the smallest this library supports)."""
    B, S, H, D = 2, 5, 2, 32
    n = B * S * H * D
    q, k, v, dy = (sdpa_inputs.hash_inputs(n, s).reshape(B, S, H, D).to(dtype) for s in (1, 2, 3, 4))
    full = gpu_run(q, k, v, dy, mask_kind="causal")
    for w, name in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        one = gpu_run(q, k, v, dy, wrt=w, mask_kind="causal")
        assert np.array_equal(one[name], full[name]), name
        for other in {"dq", "dk", "dv"} - {name}:
            assert one[other] is None
    ref = oracle_run(q, k, v, dy, mask_kind="causal")
    assert_parity(full, ref, dtype)


def test_layouts_bitwise_identical():
    """[B, S, H, D], [B, H, S, D] (as a transposed view) and a padded-stride
    layout give bit-identical gradients."""
    B, S, H, D = 2, 150, 3, 64
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=11, dtype=torch.bfloat16)
    base = gpu_run(q, k, v, dy, mask_kind="causal")
    bhsd = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v, dy)]
    r1 = gpu_run(*bhsd, mask_kind="causal")
    padded = []
    for x in (q, k, v, dy):
        big = torch.zeros(B, S, H + 1, D + 64, dtype=x.dtype)
        big[:, :, :H, :D] = x
        padded.append(big[:, :, :H, :D])
    r2 = gpu_run(*padded, mask_kind="causal")
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(base[n], r1[n]) and np.array_equal(base[n], r2[n]), n


def test_reruns_bitwise_identical_with_concurrent_work():
    import scaled_dot_product_bwd_amd as sdb
    dev = torch.device("cuda:0")
    B, S, H, D = 2, 700, 4, 128
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=3, dtype=torch.bfloat16)
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    first = [t.clone() for t in sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal")]
    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device=dev)
    for _ in range(5):
        with torch.cuda.stream(side):
            for _ in range(3):
                big = big @ big.T * 1e-3
        again = sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal")
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_validation_errors_on_device_tensors():
    import scaled_dot_product_bwd_amd as sdb
    dev = torch.device("cuda:0")
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(1, 64, 64, 2, 32, seed=1, dtype=torch.float32)
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    with pytest.raises(sdb.AttnError, match="ATTN_E_INVALID"):
        sdb.attn_bwd(qd, kd, vd, gd, out=(qd.clone(), kd, vd.clone()))  # dk aliases k
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(sdb.AttnError, match="ATTN_E_WORKSPACE"):
        sdb.attn_bwd(qd, kd, vd, gd, workspace=ws)
    with pytest.raises(sdb.AttnError, match="ATTN_E_UNSUPPORTED"):
        x = torch.randn(1, 64, 2, 48, device=dev)
        sdb.attn_bwd(x, x, x, x)


def test_side_stream_call_with_allocations_on_the_current_stream():
    """A call on a side stream while the current stream allocates and overwrites
    memory right after it returns.  The binding's own temporaries (the
    statistics workspace, the outputs, the contiguous copy of a strided
    log-sum-exp) are recorded on the side stream, so torch's allocator does not
    hand them out again before the kernels are done, and the side stream waits
    for what the current stream prepared.  Outputs must equal, bit for bit,
    the same call on the current stream."""
    import scaled_dot_product_bwd_amd as sdb
    dev = torch.device("cuda:0")
    B, S, H, D = 4, 1024, 8, 128
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=21, dtype=torch.bfloat16)
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
    (ref, ws) = sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal", return_workspace=True)
    ref = [t.clone() for t in ref]
    m, l, _ = sdb.row_stats_views(ws, B, H, S)
    lse_t = (m + torch.log(l)).transpose(1, 2).contiguous().transpose(1, 2)  # strided [B, H, Sq]
    o_stand = gd.clone()
    ref_ff = [t.clone() for t in sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal", fwd_lse=lse_t,
                                              fwd_out=o_stand)]
    torch.cuda.synchronize()
    nbytes = sdb.workspace_bytes(B, H, S)
    side = torch.cuda.Stream()
    for it in range(4):
        ff = it % 2 == 1
        kw = dict(fwd_lse=lse_t, fwd_out=o_stand) if ff else {}
        got = sdb.attn_bwd(qd, kd, vd, gd, mask_kind="causal", stream=side, **kw)
        # Same-size allocations on the current stream, written at once: they would
        # take the freed workspace / lse copy / outputs if those were not recorded.
        junk = [torch.full((nbytes // 4,), float("nan"), device=dev) for _ in range(4)]
        junk += [torch.full((B, S, H, D), float("nan"), dtype=torch.bfloat16, device=dev)
                 for _ in range(3)]
        junk.append(torch.full((B, H, S), float("nan"), device=dev))
        torch.cuda.synchronize()
        want = ref_ff if ff else ref
        for a_, b_ in zip(got, want):
            assert torch.equal(a_, b_), ("from_forward" if ff else "attn_bwd", it)
        del junk


# Narrow bands (a window of at most a quarter of the shorter sequence): the
# kernels then take their blocks short end first.  The order changes no value;
# these cases check that every block is still computed once, in the direct
# and the split forms, square and with the query rows at the end of the keys.
NARROW = [(1, 2, 600, 600, 64, 64), (1, 2, 300, 700, 64, 64), (2, 2, 520, 520, 128, 100)]


@pytest.mark.parametrize("B,H,Sq,Sk,D,window", NARROW)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("workspace", ["min", "split"])
def test_narrow_band_order(B, H, Sq, Sk, D, window, dtype, workspace):
    assert 4 * (window + 1) <= min(Sq, Sk)  # the narrow-band rule applies
    q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, Sq, Sk, H, D, seed=700 + Sq + window, dtype=dtype)
    res = gpu_run(q, k, v, dy, mask_kind="window", window=window, workspace=workspace)
    ref = oracle_run(q, k, v, dy, mask_kind="window", window=window, nthreads=2)
    print(Sq, Sk, window, workspace, assert_parity(res, ref, dtype, label=f"band w={window}"))
    again = gpu_run(q, k, v, dy, mask_kind="window", window=window, workspace=workspace)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(res[name], again[name]), name
