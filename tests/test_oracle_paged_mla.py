"""Pins of the latent (MLA) variant of the paged oracle (ruDNN 0.1.43
src/paged_attention/ordered_kernel.rs, `history_backward` with its `mla`
switch): each slot's latent row is both key and value, a position key adds
qp . kp to the score, the latent receives ds q + p dY and the position key ds qp.

Two independent references:
  * float64 autograd of the forward written directly in torch (the latent is
    indexed twice, as key and as value, so autograd sums both derivatives);
  * the standard paged oracle (pinned to the dense one) on a padded problem:
    key [c | kp], value [c | 0], query [q | qp], dY [dY | 0] -- then
    d latent = dK[:D] + dV[:D] and d kp = dK[D:].
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs

SCALE = 0.23


def _mla_workload(seed, *, heads=4, kv_heads=1, D=8, P=4, page_size=4, share=0,
                  shuffle=False, nan_unused=True, q_per_seq=5, nseq=3):
    return sdpa_inputs.paged_workload(seed=seed, nseq=nseq, len_lo=7, len_hi=30,
                                      q_per_seq=q_per_seq, page_size=page_size,
                                      unused_frac=0.3, heads=heads, kv_heads=kv_heads, D=D,
                                      dtype=torch.float64, share_prefix_pages=share,
                                      shuffle_rows=shuffle, nan_unused=nan_unused,
                                      position_dim=P)


def _kw(w):
    return dict(heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"])


def _autograd(w, causal=True):
    """Gradients of L = sum dY . O with respect to the latent and position-key
    pools, and the forward's (max, denominator, delta) per (row, head)."""
    heads, kv = w["heads"], w["kv_heads"]
    group = heads // kv
    ps = w["page_size"]
    lat = w["k_pool"].clone().nan_to_num(0.0).requires_grad_(True)
    kp = w["kp_pool"].clone().nan_to_num(0.0).requires_grad_(True)
    q, qp, dy = w["q"], w["qp"], w["dy"]
    qs, qpos = w["query_seq"].numpy(), w["query_pos"].numpy()
    bt = w["block_table"].numpy()
    stats = np.zeros((q.shape[0], heads, 3))
    loss = torch.zeros((), dtype=torch.float64)
    for s, L in enumerate(w["seq_lens"].numpy()):
        rows = np.where(qs == s)[0]
        if len(rows) == 0:
            continue
        slots = torch.tensor([int(bt[s, t // ps]) * ps + t % ps for t in range(int(L))])
        hidden = torch.zeros(len(rows), int(L), dtype=torch.bool)
        if causal:
            hidden = torch.arange(int(L))[None, :] > torch.tensor(qpos[rows])[:, None]
        for h in range(heads):
            g = h // group
            C, KP = lat[slots, g], kp[slots, g]
            sc = SCALE * (q[rows, h] @ C.T + qp[rows, h] @ KP.T)
            sc = sc.masked_fill(hidden, float("-inf"))
            Pm = torch.softmax(sc, dim=1)
            O = Pm @ C
            loss = loss + (dy[rows, h] * O).sum()
            m = sc.max(dim=1).values.detach()
            stats[rows, h, 0] = m.numpy()
            stats[rows, h, 1] = torch.exp(sc - m[:, None]).sum(1).detach().numpy()
            stats[rows, h, 2] = (dy[rows, h] * O).sum(1).detach().numpy()
    loss.backward()
    return lat.grad.numpy(), kp.grad.numpy(), stats


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads,kv_heads,share,shuffle", [(4, 1, 0, False), (6, 2, 2, True)])
def test_mla_matches_autograd(causal, heads, kv_heads, share, shuffle):
    w = _mla_workload(11, heads=heads, kv_heads=kv_heads, share=share, shuffle=shuffle,
                      nan_unused=False)
    g_lat, g_kp, st_ref = _autograd(w, causal)
    kw = _kw(w)
    stats = oracle.paged_mla_row_stats(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       causal=causal, scale=SCALE, **kw)
    np.testing.assert_allclose(stats, st_ref, rtol=1e-12, atol=1e-12)
    z_lat, z_kp = np.zeros(w["k_pool"].shape), np.zeros(w["kp_pool"].shape)
    d_lat, d_kp = oracle.paged_mla_kv_bwd(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                          stats, z_lat, z_kp, causal=causal, scale=SCALE, **kw)
    np.testing.assert_allclose(d_lat, g_lat, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(d_kp, g_kp, rtol=1e-10, atol=1e-12)
    # both derivatives of the latent matter: neither alone reproduces it
    assert np.abs(d_lat).max() > 1e-3 and np.abs(d_kp).max() > 1e-3


def test_mla_equals_padded_standard_oracle():
    """The latent variant is standard attention with key [c | kp], value
    [c | 0], query [q | qp] and dY [dY | 0]."""
    w = _mla_workload(21, heads=4, kv_heads=2, share=2, shuffle=True)
    D, P = w["D"], w["P"]
    kw = _kw(w)
    zq = torch.zeros(w["q"].shape[0], w["heads"], P, dtype=torch.float64)
    zk = torch.zeros(w["k_pool"].shape[0], w["kv_heads"], P, dtype=torch.float64)
    q2 = torch.cat([w["q"], w["qp"]], dim=2)
    k2 = torch.cat([w["k_pool"], w["kp_pool"]], dim=2)
    v2 = torch.cat([w["k_pool"], zk], dim=2)
    dy2 = torch.cat([w["dy"], zq], dim=2)
    st2 = oracle.paged_row_stats(w, q2, dy2, k2, v2, scale=SCALE, **kw)
    stats = oracle.paged_mla_row_stats(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       scale=SCALE, **kw)
    np.testing.assert_allclose(stats, st2, rtol=1e-12, atol=1e-12)
    z2 = np.zeros(k2.shape)
    dk2, dv2 = oracle.paged_kv_bwd(w, q2, dy2, k2, v2, stats, z2, z2, scale=SCALE, **kw)
    d_lat, d_kp = oracle.paged_mla_kv_bwd(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                          stats, np.zeros(w["k_pool"].shape),
                                          np.zeros(w["kp_pool"].shape), scale=SCALE, **kw)
    live = w["live_slots"].numpy()
    np.testing.assert_allclose(d_lat[live], dk2[live][..., :D] + dv2[live][..., :D],
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(d_kp[live], dk2[live][..., D:], rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(dv2[live][..., D:], 0.0)


def test_mla_unlisted_slots_kept_tails_zero():
    w = _mla_workload(31, heads=4, kv_heads=1, page_size=8)
    kw = _kw(w)
    stats = oracle.paged_mla_row_stats(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       scale=SCALE, **kw)
    s_lat = np.full(w["k_pool"].shape, 1234.5)
    s_kp = np.full(w["kp_pool"].shape, -77.25)
    d_lat, d_kp = oracle.paged_mla_kv_bwd(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                          stats, s_lat, s_kp, scale=SCALE, **kw)
    ps = w["page_size"]
    listed = {int(w["block_table"][s, p]) for s, L in enumerate(w["seq_lens"].numpy())
              for p in range((int(L) + ps - 1) // ps)}
    live = w["live_slots"].numpy()
    for pg in range(w["pool_pages"]):
        for t in range(pg * ps, (pg + 1) * ps):
            if pg not in listed:
                assert np.all(d_lat[t] == 1234.5) and np.all(d_kp[t] == -77.25)
            elif not live[t]:
                assert np.all(d_lat[t] == 0.0) and np.all(d_kp[t] == 0.0)
            else:
                assert np.all(np.isfinite(d_lat[t])) and np.all(np.isfinite(d_kp[t]))


def test_mla_zero_denominator_rows_contribute_nothing():
    w = _mla_workload(41, heads=2, kv_heads=1, nan_unused=False)
    kw = _kw(w)
    stats = oracle.paged_mla_row_stats(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       scale=SCALE, **kw)
    stats[:, :, 1] = 0.0
    d_lat, d_kp = oracle.paged_mla_kv_bwd(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                          stats, np.zeros(w["k_pool"].shape),
                                          np.zeros(w["kp_pool"].shape), scale=SCALE, **kw)
    assert np.all(d_lat == 0.0) and np.all(d_kp == 0.0)


def test_mla_without_position_keys_is_shared_key_value_attention():
    """P = 0: the latent alone is key and value; equals the standard oracle with
    V = K and dK + dV summed."""
    w = _mla_workload(51, heads=4, kv_heads=2, P=0)
    w["qp"] = torch.zeros(w["q"].shape[0], w["heads"], 0, dtype=torch.float64)
    w["kp_pool"] = torch.zeros(w["k_pool"].shape[0], w["kv_heads"], 0, dtype=torch.float64)
    kw = _kw(w)
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["k_pool"], scale=SCALE, **kw)
    z = np.zeros(w["k_pool"].shape)
    dk, dv = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["k_pool"], stats, z, z,
                                 scale=SCALE, **kw)
    d_lat, _ = oracle.paged_mla_kv_bwd(w, w["q"], w["qp"], w["dy"], w["k_pool"], w["kp_pool"],
                                       stats, z, np.zeros(w["kp_pool"].shape), scale=SCALE, **kw)
    live = w["live_slots"].numpy()
    np.testing.assert_allclose(d_lat[live], (dk + dv)[live], rtol=1e-11, atol=1e-12)
