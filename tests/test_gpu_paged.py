"""GPU parity of the paged, grouped-query history backward (attn_bwd_paged)
against the oracle (ruDNN 0.1.43 src/paged_attention/ordered_kernel.rs,
`history_backward`).

Every case runs the HIP kernel through the C ABI on seeded synthetic pools and
compares, slot by slot:
  * slots of listed pages: max|gpu - ref| / max|ref| within 2e-2 (bf16 inputs)
    or 1e-4 (fp32 inputs), per tensor;
  * tail slots of listed pages (no link reaches them): exactly +0;
  * slots of unlisted pages: the sentinel bits the pools were filled with,
    untouched (bit-exact).
Unused and tail slots of the K / V pools hold NaN, so reading one would show.
The statistics handed to the GPU are the oracle's (max, denominator, delta)
rounded to fp32; the oracle's own backward uses its float64 statistics.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs
import scaled_dot_product_bwd_amd as sb
from gpu_helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

SENTINEL_BITS = {torch.bfloat16: 0x7FC1, torch.float32: 0x7FC00001}


def _sentinel_pool(like):
    if like.dtype == torch.bfloat16:
        bits = torch.full(like.shape, SENTINEL_BITS[torch.bfloat16], dtype=torch.int16)
        return bits.view(torch.bfloat16)
    bits = torch.full(like.shape, SENTINEL_BITS[torch.float32], dtype=torch.int32)
    return bits.view(torch.float32)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def run_case(w, *, causal=True, need="dkdv", stats=None, check=True, label="", gpu_stats=None,
             kv_workgroups=0):
    """stats: the oracle's statistics (computed here when None), used by the
    reference and, rounded to fp32, by the GPU unless `gpu_stats` (a device
    tensor computed on the GPU) is given for the GPU call.  kv_workgroups:
    the dK / dV kernel form (0 automatic, n > 0 persistent with n workgroups,
    -1 one workgroup per unit)."""
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    kw = dict(heads=heads, kv_heads=kv, page_size=ps)
    if stats is None:
        stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"],
                                       causal=causal, **kw)
    plan = sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                         pool_pages=w["pool_pages"], device="cuda:0", **kw)
    print(f"[paged] {label} nq={w['q'].shape[0]} heads={heads}/{kv} D={w['D']} ps={ps} "
          f"pool={w['pool_pages']} items={plan.items} {w['dtype']} causal={causal} need={need} "
          f"kv_workgroups={kv_workgroups}", flush=True)
    dev = torch.device("cuda:0")
    st32 = gpu_stats if gpu_stats is not None else torch.from_numpy(stats.astype(np.float32)).to(dev)
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    dk0, dv0 = _sentinel_pool(w["k_pool"]), _sentinel_pool(w["v_pool"])
    dk = dk0.to(dev) if need in ("dk", "dkdv") else None
    dv = dv0.to(dev) if need in ("dv", "dkdv") else None
    sb.attn_bwd_paged(q, dy, kp, vp, st32, plan, dk_pool=dk, dv_pool=dv, need=need, causal=causal,
                      kv_workgroups=kv_workgroups)
    torch.cuda.synchronize()
    out = {"dk": None if dk is None else dk.cpu(), "dv": None if dv is None else dv.cpu(),
           "plan": plan, "stats": stats}
    if not check:
        return out
    dk_ref, dv_ref = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats,
                                         np.zeros(w["k_pool"].shape), np.zeros(w["v_pool"].shape),
                                         causal=causal, **kw)
    listed = np.zeros(w["pool_pages"] * ps, dtype=bool)
    for pg in plan.listed_pages():
        listed[pg * ps:(pg + 1) * ps] = True
    live = w["live_slots"].numpy()
    tol = TOL[w["dtype"]]
    for name, got, ref, init in (("dk", out["dk"], dk_ref, dk0), ("dv", out["dv"], dv_ref, dv0)):
        if got is None:
            continue
        g64 = got.double().numpy()
        assert not np.isnan(g64[listed]).any(), f"{label} {name}: NaN in a listed slot"
        e = rel_err(g64[listed], ref[listed])
        assert e <= tol, f"{label} {name}: rel err {e:.3e} > {tol:g}"
        gb, ib = _bits(got), _bits(init)
        assert np.array_equal(gb[~listed], ib[~listed]), f"{label} {name}: unlisted slot written"
        tail = listed & ~live
        assert (gb[tail] == 0).all(), f"{label} {name}: tail slot is not +0"
        out[name + "_err"] = e
    return out


CASES = [
    # bf16, GQA 4, shared prefix, packed rows shuffled, page 16
    dict(seed=101, nseq=3, len_lo=40, len_hi=300, q_per_seq=24, page_size=16, heads=8,
         kv_heads=2, D=128, dtype=torch.bfloat16, share_prefix_pages=3, shuffle_rows=True),
    # fp32 MHA, page 8, more rows than one chunk
    dict(seed=102, nseq=2, len_lo=60, len_hi=200, q_per_seq=40, page_size=8, heads=2,
         kv_heads=2, D=64, dtype=torch.float32),
    # bf16, pages larger than an item, GQA 2
    dict(seed=103, nseq=2, len_lo=150, len_hi=600, q_per_seq=20, page_size=256, heads=4,
         kv_heads=2, D=32, dtype=torch.bfloat16, shuffle_rows=True),
    # fp32, page size that does not divide an item, GQA 3
    dict(seed=104, nseq=3, len_lo=30, len_hi=150, q_per_seq=9, page_size=48, heads=6,
         kv_heads=2, D=128, dtype=torch.float32, share_prefix_pages=1),
    # bf16, one-token pages
    dict(seed=105, nseq=2, len_lo=10, len_hi=90, q_per_seq=7, page_size=1, heads=4,
         kv_heads=4, D=64, dtype=torch.bfloat16),
    # bf16, GQA 8, rows far from the end (a prefill chunk in the middle)
    dict(seed=106, nseq=2, len_lo=300, len_hi=700, q_per_seq=70, page_size=16, heads=16,
         kv_heads=2, D=128, dtype=torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_paged_parity(case, causal):
    w = sdpa_inputs.paged_workload(**case)
    if case["seed"] == 106:
        # queries at positions len/2 - q .. len/2: tokens past them are unseen when causal
        qp = w["query_pos"].clone()
        for s in range(len(w["seq_lens"])):
            m = w["query_seq"] == s
            qp[m] = qp[m] - int(w["seq_lens"][s]) // 2
        w["query_pos"] = qp
    run_case(w, causal=causal, label=f"seed{case['seed']}")


@pytest.mark.parametrize("need", ["dk", "dv"])
def test_paged_single_output(need):
    w = sdpa_inputs.paged_workload(seed=107, nseq=2, len_lo=50, len_hi=120, q_per_seq=12,
                                   page_size=16, heads=4, kv_heads=1, D=64, dtype=torch.bfloat16)
    run_case(w, need=need, label=f"need={need}")


def test_paged_edge_sequences():
    """A sequence without query rows and rows whose denominator is zero."""
    w = sdpa_inputs.paged_workload(seed=108, nseq=3, len_lo=40, len_hi=90, q_per_seq=6,
                                   page_size=16, heads=4, kv_heads=2, D=32, dtype=torch.float32)
    keep = w["query_seq"] != 1                      # sequence 1 has no rows: its pages get 0
    for n in ("query_seq", "query_pos", "q", "dy"):
        w[n] = w[n][keep].contiguous()
    kw = dict(heads=4, kv_heads=2, page_size=16)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    stats[0, :, 1] = 0.0                            # a row the pages skip (denominator 0)
    stats[0, :, 0] = -np.inf
    out = run_case(w, stats=stats, label="edges")
    assert out["dk_err"] <= TOL[torch.float32]


def test_paged_config5_full():
    """16 sequences of UniformInt[256, 4096] tokens, 32 / 8 heads, D 128, page 16,
    64 queries per sequence at its last positions, 25% unused pool pages, bf16,
    every listed slot against the oracle (the form the library picks: the
    persistent one on a GPU with fewer compute units than the 2648 units);
    then a rerun of that form and a run of the one-workgroup-per-unit form,
    all bit-identical."""
    w = sdpa_inputs.paged_workload(seed=1005)
    out = run_case(w, label="config5")
    print(f"[paged] config5 rel err dk {out['dk_err']:.3e} dv {out['dv_err']:.3e}", flush=True)
    again = run_case(w, stats=out["stats"], check=False, label="config5 rerun")
    assert torch.equal(_bits_t(out["dk"]), _bits_t(again["dk"]))
    assert torch.equal(_bits_t(out["dv"]), _bits_t(again["dv"]))
    classic = run_case(w, stats=out["stats"], check=False, label="config5 per-unit form",
                       kv_workgroups=-1)
    assert torch.equal(_bits_t(out["dk"]), _bits_t(classic["dk"]))
    assert torch.equal(_bits_t(out["dv"]), _bits_t(classic["dv"]))


FORM_CASES = [c for c in CASES if c["dtype"] == torch.bfloat16] + [
    # many items per workgroup, 16 queries per sequence (one-chunk links), GQA 4
    dict(seed=110, nseq=6, len_lo=64, len_hi=900, q_per_seq=4, page_size=16, heads=8,
         kv_heads=2, D=64, dtype=torch.bfloat16),
    # many items per workgroup with two- and three-chunk links (unit switches
    # while the next link's first two chunks are in flight), D 128
    dict(seed=112, nseq=3, len_lo=300, len_hi=900, q_per_seq=32, page_size=16, heads=8,
         kv_heads=2, D=128, dtype=torch.bfloat16),
    dict(seed=113, nseq=3, len_lo=300, len_hi=900, q_per_seq=48, page_size=16, heads=8,
         kv_heads=2, D=128, dtype=torch.bfloat16),
]


@pytest.mark.parametrize("case", FORM_CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("wgs", [8, 16])
def test_paged_persistent_form(case, causal, wgs):
    """The persistent form with few workgroups (so each walks many units, links
    and unit switches) against the oracle, and bit-identical to the
    one-workgroup-per-unit form, on the full pools (unlisted slots untouched,
    tail slots +0)."""
    w = sdpa_inputs.paged_workload(**case)
    if case["seed"] == 106:
        qp = w["query_pos"].clone()
        for s in range(len(w["seq_lens"])):
            m = w["query_seq"] == s
            qp[m] = qp[m] - int(w["seq_lens"][s]) // 2
        w["query_pos"] = qp
    label = f"seed{case['seed']} wgs={wgs}"
    out = run_case(w, causal=causal, label=label, kv_workgroups=wgs)
    ref = run_case(w, causal=causal, stats=out["stats"], check=False, label=label + " per-unit",
                   kv_workgroups=-1)
    for name in ("dk", "dv"):
        assert torch.equal(_bits_t(out[name]), _bits_t(ref[name])), f"{label} {name}"


@pytest.mark.parametrize("need", ["dk", "dv"])
def test_paged_persistent_single_output_and_empty_units(need):
    """One gradient only, a sequence without query rows (its units store
    zeros from the persistent form's scan) and a zero-denominator row."""
    w = sdpa_inputs.paged_workload(seed=111, nseq=4, len_lo=40, len_hi=400, q_per_seq=10,
                                   page_size=16, heads=4, kv_heads=2, D=128, dtype=torch.bfloat16)
    keep = w["query_seq"] != 2
    for n in ("query_seq", "query_pos", "q", "dy"):
        w[n] = w[n][keep].contiguous()
    kw = dict(heads=4, kv_heads=2, page_size=16)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    stats[0, :, 1] = 0.0
    stats[0, :, 0] = -np.inf
    out = run_case(w, stats=stats, need=need, label=f"persistent need={need}", kv_workgroups=8)
    ref = run_case(w, stats=stats, need=need, check=False, label="per-unit", kv_workgroups=-1)
    assert torch.equal(_bits_t(out[need]), _bits_t(ref[need]))


def _bits_t(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def test_paged_rejections():
    w = sdpa_inputs.paged_workload(seed=109, nseq=2, len_lo=20, len_hi=40, q_per_seq=4,
                                   page_size=16, heads=4, kv_heads=2, D=64, dtype=torch.bfloat16)
    plan = sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                         heads=4, kv_heads=2, page_size=16, pool_pages=w["pool_pages"],
                         device="cuda:0")
    dev = torch.device("cuda:0")
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    st = torch.ones(q.shape[0], 4, 3, device=dev)
    dk = torch.zeros_like(kp)
    with pytest.raises(sb.AttnError, match="INVALID"):   # output aliases an input
        sb.attn_bwd_paged(q, dy, kp, vp, st, plan, dk_pool=kp, need="dk")
    with pytest.raises(sb.AttnError, match="UNSUPPORTED"):  # head_dim 48
        sb.attn_bwd_paged(q[..., :48].contiguous(), dy[..., :48].contiguous(),
                          kp[..., :48].contiguous(), vp[..., :48].contiguous(), st, plan,
                          dk_pool=dk[..., :48].contiguous(), need="dk")
    with pytest.raises(sb.AttnError, match="kv_workgroups"):
        sb.attn_bwd_paged(q, dy, kp, vp, st, plan, dk_pool=dk, need="dk", kv_workgroups=-2)
    bad = sb.PagedPlan(plan.words.copy(), heads=4, kv_heads=2, page_size=16,
                       pool_pages=w["pool_pages"], nq=plan.nq, device=dev)
    bad.words[0] ^= 1
    with pytest.raises(sb.AttnError, match="magic"):
        sb.attn_bwd_paged(q, dy, kp, vp, st, bad, dk_pool=dk, need="dk")
    other = sb.PagedPlan(plan.words, heads=8, kv_heads=2, page_size=16,
                         pool_pages=w["pool_pages"], nq=plan.nq, device=dev)
    q8 = torch.zeros(q.shape[0], 8, 64, dtype=q.dtype, device=dev)
    with pytest.raises(sb.AttnError, match="plan was built"):
        sb.attn_bwd_paged(q8, q8, kp, vp, torch.ones(q.shape[0], 8, 3, device=dev), other,
                          dk_pool=dk, need="dk")
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0                   # nothing ran


# ---------------------------------------------------------------------------
# Query side: statistics and dQ (attn_bwd_paged_row_stats, attn_bwd_paged_dq).

def _stats_err(got, ref):
    """Per component (max, denominator, delta) over the rows that see a token."""
    fin = ref[..., 1] > 0
    errs = []
    for k in range(3):
        errs.append(rel_err(got[..., k][fin], ref[..., k][fin]))
    empty = ~fin
    assert np.all(np.isneginf(got[..., 0][empty])) and np.all(got[..., 1:][empty] == 0)
    return errs


def run_query_side(w, *, causal=True, label="", split=True):
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    kw = dict(heads=heads, kv_heads=kv, page_size=ps)
    plan = sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                         pool_pages=w["pool_pages"], device="cuda:0", **kw)
    print(f"[paged-q] {label} nq={w['q'].shape[0]} heads={heads}/{kv} D={w['D']} ps={ps} "
          f"{w['dtype']} causal={causal} qblocks={plan.header(sb._abi.W_QBLK)} "
          f"pieces={plan.header(sb._abi.W_QPIECES)} split={split}", flush=True)
    dev = torch.device("cuda:0")
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    st_gpu = sb.paged_row_stats(q, dy, kp, vp, plan, causal=causal, split=split)
    st_ref = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], causal=causal, **kw)
    # dQ from the oracle's statistics (rounded to fp32), against the oracle's dQ
    st32 = torch.from_numpy(st_ref.astype(np.float32)).to(dev)
    dq_gpu = sb.attn_bwd_paged_dq(q, dy, kp, vp, st32, plan, causal=causal, split=split)
    torch.cuda.synchronize()
    dq_ref = oracle.paged_dq(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], st_ref, causal=causal, **kw)
    tol = TOL[w["dtype"]]
    errs = _stats_err(st_gpu.cpu().double().numpy(), st_ref)
    for name, e in zip(("max", "denominator", "delta"), errs):
        assert e <= tol, f"{label} stats {name}: rel err {e:.3e} > {tol:g}"
    g = dq_gpu.double().cpu().numpy()
    assert not np.isnan(g).any()
    e = rel_err(g, dq_ref)
    assert e <= tol, f"{label} dq: rel err {e:.3e} > {tol:g}"
    # Both in one call (attn_bwd_paged_stats_dq), against the same oracle values.
    st_f, dq_f = sb.paged_stats_dq(q, dy, kp, vp, plan, causal=causal,
                                   form="split" if split else "direct")
    torch.cuda.synchronize()
    errs_f = _stats_err(st_f.cpu().double().numpy(), st_ref)
    for name, ef in zip(("max", "denominator", "delta"), errs_f):
        assert ef <= tol, f"{label} fused stats {name}: rel err {ef:.3e} > {tol:g}"
    gf = dq_f.double().cpu().numpy()
    assert not np.isnan(gf).any()
    empty = st_ref[..., 1] == 0
    assert (gf[empty] == 0).all(), f"{label} fused dq: a row that sees nothing is not zero"
    e_f = rel_err(gf, dq_ref)
    assert e_f <= tol, f"{label} fused dq: rel err {e_f:.3e} > {tol:g}"
    return dict(plan=plan, stats=st_gpu, dq=dq_gpu, stats_err=errs, dq_err=e, st32=st32,
                fused_stats=st_f, fused_dq=dq_f, fused_stats_err=errs_f, fused_dq_err=e_f)


# Sequences longer than a 1024-token piece, so the split form merges several
# pieces per query block (seed 110: queries in the middle, so under the causal
# mask the pieces past them see nothing).
LONG_CASES = [
    dict(seed=109, nseq=3, len_lo=1100, len_hi=2700, q_per_seq=20, page_size=16, heads=8,
         kv_heads=2, D=64, dtype=torch.bfloat16, shuffle_rows=True),
    dict(seed=110, nseq=2, len_lo=2100, len_hi=3300, q_per_seq=36, page_size=32, heads=4,
         kv_heads=1, D=128, dtype=torch.float32),
]
Q_CASES = [CASES[0], CASES[1], CASES[2], CASES[3], CASES[4], CASES[5]] + LONG_CASES


def _middle_rows(w):
    qp = w["query_pos"].clone()
    for s in range(len(w["seq_lens"])):
        m = w["query_seq"] == s
        qp[m] = qp[m] - int(w["seq_lens"][s]) // 2
    w["query_pos"] = qp


@pytest.mark.parametrize("case", Q_CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("split", [True, False], ids=["split", "direct"])
def test_paged_query_side_parity(case, causal, split):
    w = sdpa_inputs.paged_workload(**case)
    if case["seed"] in (106, 110):
        _middle_rows(w)
    run_query_side(w, causal=causal, label=f"seed{case['seed']}", split=split)


def test_paged_query_split_rerun_bitwise():
    """The split form's merge runs in a fixed piece order: reruns are bit-identical
    (the separate calls and the fused one)."""
    w = sdpa_inputs.paged_workload(**LONG_CASES[0])
    out = run_query_side(w, label="rerun")
    dev = torch.device("cuda:0")
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    st2 = sb.paged_row_stats(q, dy, kp, vp, out["plan"])
    dq2 = sb.attn_bwd_paged_dq(q, dy, kp, vp, out["st32"], out["plan"])
    st3, dq3 = sb.paged_stats_dq(q, dy, kp, vp, out["plan"], form="split")
    torch.cuda.synchronize()
    assert torch.equal(st2.view(torch.int32), out["stats"].view(torch.int32))
    assert torch.equal(dq2.view(torch.int16), out["dq"].view(torch.int16))
    assert torch.equal(st3.view(torch.int32), out["fused_stats"].view(torch.int32))
    assert torch.equal(dq3.view(torch.int16), out["fused_dq"].view(torch.int16))


@pytest.mark.parametrize("split", [True, False], ids=["split", "direct"])
def test_paged_query_side_edges(split):
    """A sequence of length 0 that has query rows (statistics (-inf, 0, 0), zero
    dQ rows), rows at positions past their sequence's end (they see all of it),
    a single-token sequence, bf16 and fp32."""
    for dtype, D in ((torch.bfloat16, 64), (torch.float32, 32)):
        w = sdpa_inputs.paged_workload(seed=114, nseq=4, len_lo=70, len_hi=260, q_per_seq=10,
                                       page_size=16, heads=4, kv_heads=2, D=D, dtype=dtype)
        lens = w["seq_lens"].clone()
        lens[1] = 0
        lens[3] = 1
        w["seq_lens"] = lens
        qp = w["query_pos"].clone()
        qp[w["query_seq"] == 2] += 50
        w["query_pos"] = qp
        for causal in (True, False):
            run_query_side(w, causal=causal, label=f"edges {dtype} causal={causal}", split=split)


def test_paged_config5_gpu_chain():
    """Config 5 with no precomputed statistics: GPU statistics -> GPU dK / dV and
    GPU dQ, against the oracle run end to end in float64."""
    w = sdpa_inputs.paged_workload(seed=1005)
    out = run_query_side(w, label="config5")
    print(f"[paged-q] config5 stats err {out['stats_err']} dq err {out['dq_err']:.3e} fused "
          f"{out['fused_stats_err']} {out['fused_dq_err']:.3e}", flush=True)
    # the fused call's library-picked form gives the bits of one of the two forms
    dev = torch.device("cuda:0")
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    st_d, dq_d = sb.paged_stats_dq(q, dy, kp, vp, out["plan"], form="direct")
    st_a, dq_a = sb.paged_stats_dq(q, dy, kp, vp, out["plan"], form="auto")
    torch.cuda.synchronize()
    same = [torch.equal(st_a.view(torch.int32), x.view(torch.int32)) and
            torch.equal(dq_a.view(torch.int16), y.view(torch.int16))
            for x, y in ((st_d, dq_d), (out["fused_stats"], out["fused_dq"]))]
    assert any(same), "the picked form matches neither form bitwise"
    print(f"[paged-q] config5 fused form picked: {'direct' if same[0] else 'split'}", flush=True)
    kv = run_case(w, gpu_stats=out["stats"], label="config5 gpu-stats")
    print(f"[paged-q] config5 chain dk {kv['dk_err']:.3e} dv {kv['dv_err']:.3e}", flush=True)
