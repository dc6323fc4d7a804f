"""Pins of the paged oracle (ruDNN 0.1.43 src/paged_attention/ordered_kernel.rs,
`history_backward`) to the dense oracle, which is itself pinned in test_oracle.py.

A sequence's history gathered through its block table is an ordinary dense
causal problem whose queries are the last rows (offset len - rows); each KV head
serves `heads / kv_heads` query heads, so a slot's dK / dV is the dense dK / dV
summed over the group's heads and over every (sequence, logical page) that maps
to the slot.  Slots of pages no sequence lists keep the caller's contents; slots
past a sequence's end on a listed page get zero.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs


def _dense_reference(w):
    heads, kv, ps, D = w["heads"], w["kv_heads"], w["page_size"], w["D"]
    group = heads // kv
    q, dy = w["q"].double().numpy(), w["dy"].double().numpy()
    kp, vp = w["k_pool"].double().numpy(), w["v_pool"].double().numpy()
    nslot = kp.shape[0]
    dk = np.zeros((nslot, kv, D))
    dv = np.zeros((nslot, kv, D))
    dq = np.zeros(q.shape)
    stats = np.zeros((q.shape[0], heads, 3))
    qs, qpos = w["query_seq"].numpy(), w["query_pos"].numpy()
    bt = w["block_table"].numpy()
    for s, L in enumerate(w["seq_lens"].numpy()):
        rows = np.where(qs == s)[0]
        rows = rows[np.argsort(qpos[rows])]
        assert np.array_equal(qpos[rows], np.arange(L - len(rows), L))
        slots = np.array([bt[s, t // ps] * ps + t % ps for t in range(L)])
        heads_of = np.arange(heads) // group
        Kd = kp[slots][:, heads_of][None]   # [1, L, heads, D]
        Vd = vp[slots][:, heads_of][None]
        r = oracle.attn_bwd(q[rows][None], Kd, Vd, dy[rows][None],
                            mask_kind=oracle.MASK_CAUSAL)
        for g in range(kv):
            hs = slice(g * group, (g + 1) * group)
            np.add.at(dk, (slots, g), r["dk"][0][:, hs].sum(1))
            np.add.at(dv, (slots, g), r["dv"][0][:, hs].sum(1))
        stats[rows, :, 0] = r["m"][0].T
        stats[rows, :, 1] = r["l"][0].T
        stats[rows, :, 2] = r["delta"][0].T
        dq[rows] = r["dq"][0]
    _dense_reference.dq = dq
    return dk, dv, stats


def _listed_pages(w):
    ps = w["page_size"]
    out = set()
    for s, L in enumerate(w["seq_lens"].numpy()):
        for p in range((int(L) + ps - 1) // ps):
            out.add(int(w["block_table"][s, p]))
    return out


@pytest.mark.parametrize("share,shuffle", [(0, False), (3, False), (2, True)])
def test_paged_equals_dense_gather_scatter(share, shuffle):
    w = sdpa_inputs.paged_workload(seed=7, nseq=3, len_lo=9, len_hi=40, q_per_seq=6,
                                   page_size=4, unused_frac=0.3, heads=4, kv_heads=2, D=8,
                                   dtype=torch.float64, share_prefix_pages=share,
                                   shuffle_rows=shuffle)
    kw = dict(heads=4, kv_heads=2, page_size=4)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    dk_ref, dv_ref, st_ref = _dense_reference(w)
    np.testing.assert_allclose(stats, st_ref, rtol=1e-12, atol=1e-12)

    sentinel = np.full(w["k_pool"].shape, 1234.5)
    dk, dv = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats,
                                 sentinel, sentinel, **kw)
    listed = _listed_pages(w)
    ps = w["page_size"]
    live = w["live_slots"].numpy()
    for pg in range(w["pool_pages"]):
        sl = slice(pg * ps, (pg + 1) * ps)
        if pg not in listed:
            assert np.all(dk[sl] == 1234.5) and np.all(dv[sl] == 1234.5)
            continue
        np.testing.assert_allclose(dk[sl], dk_ref[sl], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dv[sl], dv_ref[sl], rtol=1e-11, atol=1e-11)
        for t in range(pg * ps, (pg + 1) * ps):
            if not live[t]:
                assert np.all(dk[t] == 0.0) and np.all(dv[t] == 0.0)
    if share:
        # a shared page really has several contributors: dropping the second
        # sequence changes its gradient
        assert len(listed) < sum((int(L) + ps - 1) // ps for L in w["seq_lens"])


def test_paged_grouping_reduces_to_mha():
    """heads == kv_heads: every KV head serves exactly one query head."""
    w = sdpa_inputs.paged_workload(seed=3, nseq=2, len_lo=5, len_hi=20, q_per_seq=4,
                                   page_size=2, heads=3, kv_heads=3, D=4, dtype=torch.float64)
    kw = dict(heads=3, kv_heads=3, page_size=2)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    z = np.zeros(w["k_pool"].shape)
    dk, dv = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats, z, z, **kw)
    dk_ref, dv_ref, _ = _dense_reference(w)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-11, atol=1e-11)


def test_paged_zero_denominator_rows_contribute_nothing():
    """Rows whose statistics carry denominator 0 are skipped (history_backward
    tests `denominator != 0` before any contribution)."""
    w = sdpa_inputs.paged_workload(seed=5, nseq=2, len_lo=8, len_hi=16, q_per_seq=3,
                                   page_size=4, heads=2, kv_heads=1, D=4, dtype=torch.float64)
    kw = dict(heads=2, kv_heads=1, page_size=4)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    z = np.zeros(w["k_pool"].shape)
    stats0 = stats.copy()
    stats0[:, :, 1] = 0.0
    dk, dv = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats0, z, z, **kw)
    assert np.all(dk == 0) and np.all(dv == 0)
    # only sequence 1's rows zeroed: sequence 0's pages keep their gradient
    stats1 = stats.copy()
    stats1[w["query_seq"].numpy() == 1, :, 1] = 0.0
    dk1, _ = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats1, z, z, **kw)
    dkf, _ = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats, z, z, **kw)
    bt, ps = w["block_table"].numpy(), 4
    L0 = int(w["seq_lens"][0])
    s0 = [bt[0, t // ps] * ps + t % ps for t in range(L0)]
    np.testing.assert_allclose(dk1[s0], dkf[s0], rtol=1e-14)


def test_paged_rejects_bad_tables():
    w = sdpa_inputs.paged_workload(seed=1, nseq=1, len_lo=4, len_hi=4, q_per_seq=2,
                                   page_size=2, heads=2, kv_heads=1, D=4, dtype=torch.float64)
    w["block_table"][0, 0] = 10_000
    with pytest.raises(ValueError):
        oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], heads=2,
                               kv_heads=1, page_size=2)


@pytest.mark.parametrize("share,shuffle", [(0, False), (2, True)])
def test_paged_dq_equals_dense_gather(share, shuffle):
    """dQ of each packed row equals the dense oracle's dQ on its gathered
    sequence (causal offset len - rows), with the oracle's own statistics."""
    w = sdpa_inputs.paged_workload(seed=17, nseq=3, len_lo=9, len_hi=40, q_per_seq=6,
                                   page_size=4, heads=4, kv_heads=2, D=8, dtype=torch.float64,
                                   share_prefix_pages=share, shuffle_rows=shuffle)
    kw = dict(heads=4, kv_heads=2, page_size=4)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    dq = oracle.paged_dq(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats, **kw)
    _dense_reference(w)
    np.testing.assert_allclose(dq, _dense_reference.dq, rtol=1e-11, atol=1e-11)
    # a row the pages skip (zero denominator) gets a zero dQ row
    st0 = stats.copy()
    st0[1, :, 1] = 0.0
    dq0 = oracle.paged_dq(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], st0, **kw)
    assert np.all(dq0[1] == 0.0)
    np.testing.assert_array_equal(dq0[0], dq[0])
