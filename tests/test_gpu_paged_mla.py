"""GPU parity of the latent (MLA) variant of the paged history backward
(attn_bwd_paged with mla = 1) against the oracle (ruDNN 0.1.43
src/paged_attention/ordered_kernel.rs, `history_backward`, its `mla` switch).

Each slot's latent row is both key and value; a position key adds qp . kp to
the score.  Per case, slot by slot, for the latent's gradient and the position
keys' gradient:
  * slots of listed pages: max|gpu - ref| / max|ref| within 2e-2 (bf16 inputs)
    or 1e-4 (fp32 inputs), per tensor;
  * tail slots of listed pages: exactly +0;
  * slots of unlisted pages: the sentinel bits, untouched (bit-exact).
Unused and tail slots of the latent and position-key pools hold NaN.  The GPU
gets the oracle's statistics rounded to fp32; the oracle uses its float64 ones.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs
import scaled_dot_product_bwd_amd as sb
from gpu_helpers import TOL, rel_err
from test_gpu_paged import _bits, _sentinel_pool

pytestmark = pytest.mark.gpu


def _scale(w):
    return float(np.float32(1.0) / np.sqrt(np.float32(w["D"] + w["P"])))


def run_mla(w, *, causal=True, need="both", label="", compare_seqs=None, stats=None):
    """compare_seqs: compare only the slots of these sequences (the oracle then
    runs on those sequences alone: without shared pages, a slot's gradient
    depends only on its own sequence's rows)."""
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    kw = dict(heads=heads, kv_heads=kv, page_size=ps)
    scale = _scale(w)
    wr = w
    if compare_seqs is not None:
        keep = np.isin(w["query_seq"].numpy(), compare_seqs)
        wr = dict(w)
        sel = torch.from_numpy(np.asarray(compare_seqs, dtype=np.int64))
        remap = {int(s): i for i, s in enumerate(compare_seqs)}
        wr["seq_lens"] = w["seq_lens"][sel]
        wr["block_table"] = w["block_table"][sel]
        kt = torch.from_numpy(keep)
        wr["query_seq"] = torch.tensor([remap[int(s)] for s in w["query_seq"][kt]], dtype=torch.int32)
        for n in ("query_pos", "q", "qp", "dy"):
            wr[n] = w[n][kt]
    if stats is None:
        stats = oracle.paged_mla_row_stats(wr, wr["q"], wr["qp"], wr["dy"], w["k_pool"],
                                           w["kp_pool"], causal=causal, scale=scale, **kw)
    # GPU statistics: the oracle's rows where compared, the rest from a cheap
    # stand-in (finite, positive denominators; those slots are not compared)
    nq = w["q"].shape[0]
    st_gpu = np.zeros((nq, heads, 3))
    st_gpu[:, :, 0] = 3.0
    st_gpu[:, :, 1] = 1e3
    if compare_seqs is None:
        st_gpu[:] = stats
    else:
        st_gpu[keep] = stats
    plan = sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                         pool_pages=w["pool_pages"], device="cuda:0", **kw)
    print(f"[mla] {label} nq={nq} heads={heads}/{kv} D={w['D']} P={w['P']} ps={ps} "
          f"pool={w['pool_pages']} items={plan.items} {w['dtype']} causal={causal} need={need}",
          flush=True)
    dev = torch.device("cuda:0")
    st32 = torch.from_numpy(st_gpu.astype(np.float32)).to(dev)
    q, qp, dy, lat, kpp = (w[n].to(dev) for n in ("q", "qp", "dy", "k_pool", "kp_pool"))
    l0, p0 = _sentinel_pool(w["k_pool"]), _sentinel_pool(w["kp_pool"])
    dl = l0.to(dev) if need in ("dlat", "both") else None
    dp = p0.to(dev) if need in ("dkp", "both") and w["P"] > 0 else None
    sb.attn_bwd_paged_mla(q, qp, dy, lat, kpp, st32, plan, dlat_pool=dl, dkp_pool=dp, need=need,
                          causal=causal, scale=scale)
    torch.cuda.synchronize()
    out = {"dlat": None if dl is None else dl.cpu(), "dkp": None if dp is None else dp.cpu(),
           "plan": plan, "stats": stats, "st32": st32}
    r_lat, r_kp = oracle.paged_mla_kv_bwd(wr, wr["q"], wr["qp"], wr["dy"], w["k_pool"],
                                          w["kp_pool"], stats, np.zeros(w["k_pool"].shape),
                                          np.zeros(w["kp_pool"].shape), causal=causal,
                                          scale=scale, **kw)
    listed = np.zeros(w["pool_pages"] * ps, dtype=bool)
    for pg in plan.listed_pages():
        listed[pg * ps:(pg + 1) * ps] = True
    live = w["live_slots"].numpy()
    cmp = listed.copy()
    if compare_seqs is not None:
        cmp[:] = False
        bt = w["block_table"].numpy()
        for s in compare_seqs:
            for pgi in range((int(w["seq_lens"][s]) + ps - 1) // ps):
                pg = int(bt[s, pgi])
                cmp[pg * ps:(pg + 1) * ps] = True
    tol = TOL[w["dtype"]]
    for name, got, ref, init in (("dlat", out["dlat"], r_lat, l0), ("dkp", out["dkp"], r_kp, p0)):
        if got is None:
            continue
        g64 = got.double().numpy()
        assert not np.isnan(g64[listed]).any(), f"{label} {name}: NaN in a listed slot"
        e = rel_err(g64[cmp], ref[cmp])
        assert e <= tol, f"{label} {name}: rel err {e:.3e} > {tol:g}"
        gb, ib = _bits(got), _bits(init)
        assert np.array_equal(gb[~listed], ib[~listed]), f"{label} {name}: unlisted slot written"
        tail = listed & ~live
        assert (gb[tail] == 0).all(), f"{label} {name}: tail slot is not +0"
        out[name + "_err"] = e
    return out


CASES = [
    # bf16, latent 128 + position 64, one KV head for 16 query heads, shared prefix
    dict(seed=301, nseq=3, len_lo=40, len_hi=300, q_per_seq=24, page_size=16, heads=16,
         kv_heads=1, D=128, position_dim=64, dtype=torch.bfloat16, share_prefix_pages=3,
         shuffle_rows=True),
    # fp32, latent 64 + 32, GQA 2, page 8, more rows than one chunk
    dict(seed=302, nseq=2, len_lo=60, len_hi=200, q_per_seq=40, page_size=8, heads=4,
         kv_heads=2, D=64, position_dim=32, dtype=torch.float32),
    # bf16, latent 64 + 64, pages larger than an item
    dict(seed=303, nseq=2, len_lo=150, len_hi=600, q_per_seq=20, page_size=256, heads=8,
         kv_heads=1, D=64, position_dim=64, dtype=torch.bfloat16, shuffle_rows=True),
    # fp32, latent 128 + 64, page 48 (does not divide an item)
    dict(seed=304, nseq=3, len_lo=30, len_hi=150, q_per_seq=9, page_size=48, heads=4,
         kv_heads=1, D=128, position_dim=64, dtype=torch.float32, share_prefix_pages=1),
    # bf16, latent 128 + 32, one-token pages, GQA 4
    dict(seed=305, nseq=2, len_lo=10, len_hi=90, q_per_seq=7, page_size=1, heads=8,
         kv_heads=2, D=128, position_dim=32, dtype=torch.bfloat16),
    # fp32, latent 128 + 32
    dict(seed=306, nseq=2, len_lo=40, len_hi=120, q_per_seq=11, page_size=16, heads=2,
         kv_heads=1, D=128, position_dim=32, dtype=torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_mla_parity(case, causal):
    run_mla(sdpa_inputs.paged_workload(**case), causal=causal, label=f"seed{case['seed']}")


# Latents wider than 128 (bf16; 32-row chunks): rows of several chunks, shared
# prefixes, pages larger or smaller than an item, GQA.
WIDE_CASES = [
    dict(seed=310, nseq=3, len_lo=40, len_hi=300, q_per_seq=24, page_size=16, heads=8,
         kv_heads=1, D=256, position_dim=64, dtype=torch.bfloat16, share_prefix_pages=2,
         shuffle_rows=True),
    dict(seed=311, nseq=2, len_lo=60, len_hi=200, q_per_seq=13, page_size=48, heads=4,
         kv_heads=2, D=192, position_dim=32, dtype=torch.bfloat16),
    dict(seed=312, nseq=2, len_lo=10, len_hi=90, q_per_seq=7, page_size=1, heads=4,
         kv_heads=1, D=256, position_dim=32, dtype=torch.bfloat16),
    dict(seed=313, nseq=2, len_lo=100, len_hi=300, q_per_seq=40, page_size=256, heads=8,
         kv_heads=2, D=192, position_dim=64, dtype=torch.bfloat16, shuffle_rows=True),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_mla_wide_latent_parity(case, causal):
    run_mla(sdpa_inputs.paged_workload(**case), causal=causal, label=f"seed{case['seed']}")


@pytest.mark.parametrize("D,dtype", [(64, torch.bfloat16), (128, torch.float32),
                                     (128, torch.bfloat16), (192, torch.bfloat16),
                                     (256, torch.bfloat16)])
def test_mla_without_position_keys(D, dtype):
    """P = 0: the latent alone is key and value."""
    w = sdpa_inputs.paged_workload(seed=307, nseq=2, len_lo=50, len_hi=160, q_per_seq=30,
                                   page_size=16, heads=4, kv_heads=1, D=D, dtype=dtype)
    nq = w["q"].shape[0]
    w["qp"] = torch.zeros(nq, 4, 0, dtype=dtype)
    w["kp_pool"] = torch.zeros(w["k_pool"].shape[0], 1, 0, dtype=dtype)
    w["P"] = 0
    run_mla(w, need="dlat", label=f"P0 D{D}")


@pytest.mark.parametrize("need", ["dlat", "dkp"])
def test_mla_single_output(need):
    w = sdpa_inputs.paged_workload(seed=308, nseq=2, len_lo=50, len_hi=120, q_per_seq=12,
                                   page_size=16, heads=8, kv_heads=1, D=128, position_dim=64,
                                   dtype=torch.bfloat16)
    run_mla(w, need=need, label=f"need={need}")


def test_mla_middle_queries_and_zero_denominator():
    """Queries in the middle of their sequence (later tokens unseen when causal)
    and rows whose denominator is zero (skipped)."""
    w = sdpa_inputs.paged_workload(seed=309, nseq=2, len_lo=300, len_hi=500, q_per_seq=70,
                                   page_size=16, heads=8, kv_heads=1, D=128, position_dim=64,
                                   dtype=torch.bfloat16)
    qp = w["query_pos"].clone()
    for s in range(len(w["seq_lens"])):
        m = w["query_seq"] == s
        qp[m] = qp[m] - int(w["seq_lens"][s]) // 2
    w["query_pos"] = qp
    kw = dict(heads=8, kv_heads=1, page_size=16)
    stats = oracle.paged_mla_row_stats(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       scale=_scale(w), **kw)
    stats[::3, :, 1] = 0.0
    run_mla(w, stats=stats, label="middle+zero-den")


def test_mla_full_size_sampled_and_rerun_bitwise():
    """The paged workload's shape with a latent key (16 sequences of 256..4096
    tokens, 64 queries each at the end, page 16, 25% unused pages, bf16) with
    16 query heads on one latent KV head of width 128 + 64.  The oracle runs on
    two sampled sequences (no shared pages: a slot's gradient depends only on
    its sequence); a second GPU call must be bit-identical."""
    w = sdpa_inputs.paged_workload(seed=1005, heads=16, kv_heads=1, D=128, position_dim=64)
    out = run_mla(w, label="full", compare_seqs=[3, 11])
    dev = torch.device("cuda:0")
    q, qp, dy, lat, kpp = (w[n].to(dev) for n in ("q", "qp", "dy", "k_pool", "kp_pool"))
    dl = _sentinel_pool(w["k_pool"]).to(dev)
    dp = _sentinel_pool(w["kp_pool"]).to(dev)
    sb.attn_bwd_paged_mla(q, qp, dy, lat, kpp, out["st32"], out["plan"], dlat_pool=dl,
                          dkp_pool=dp, scale=_scale(w))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dl.cpu()), _bits(out["dlat"]))
    assert np.array_equal(_bits(dp.cpu()), _bits(out["dkp"]))


def test_mla_wide_full_size_sampled_and_rerun_bitwise():
    """The paged workload's shape with 16 query heads on one latent KV head of
    width 256 + 64 (bf16): two sampled sequences against the oracle, and a
    second GPU call bit-identical."""
    w = sdpa_inputs.paged_workload(seed=1005, heads=16, kv_heads=1, D=256, position_dim=64)
    out = run_mla(w, label="full wide", compare_seqs=[5, 12])
    dev = torch.device("cuda:0")
    q, qp, dy, lat, kpp = (w[n].to(dev) for n in ("q", "qp", "dy", "k_pool", "kp_pool"))
    dl = _sentinel_pool(w["k_pool"]).to(dev)
    dp = _sentinel_pool(w["kp_pool"]).to(dev)
    sb.attn_bwd_paged_mla(q, qp, dy, lat, kpp, out["st32"], out["plan"], dlat_pool=dl,
                          dkp_pool=dp, scale=_scale(w))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dl.cpu()), _bits(out["dlat"]))
    assert np.array_equal(_bits(dp.cpu()), _bits(out["dkp"]))
