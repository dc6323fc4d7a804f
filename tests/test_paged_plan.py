"""Host planner of the paged backward (attn_bwd_paged_plan_build), CPU only.

The plan regroups the tables ruDNN 0.1.43 src/paged_attention/ordered_kernel.rs
`history_backward` walks (history pages, page -> (sequence, logical page)
links, sequence -> query rows) into 128-slot items.  Two checks pin it:

* a brute-force walk in the pages' loop order (listed page -> slot -> link ->
  row of the linked sequence -> query head of the group) and the plan must
  name exactly the same written slots, the same live / tail slots and the
  same (slot, sequence, token, row, head) contributions (bit-exact, as sets);
* dK / dV evaluated in float64 from nothing but the plan tables (the way the
  kernel reads them) must equal the paged oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs
import scaled_dot_product_bwd_amd as sb
from scaled_dot_product_bwd_amd import _abi

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(sb.library_path()),
                                reason="libattn_bwd.so not built")


def _plan(w):
    return sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                         heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"],
                         pool_pages=w["pool_pages"])


def _tables(plan):
    W = plan.words
    h = lambda k: int(W[k])
    items, links, nseq, qh = h(_abi.W_ITEMS), h(_abi.W_LINKS), h(_abi.W_NSEQ), h(_abi.W_QH)
    S = _abi.PLAN_ITEM_SLOTS
    t = dict(
        item_links=W[h(_abi.W_OFF_ITEM_LINKS):][:items + 1],
        item_slots=W[h(_abi.W_OFF_ITEM_SLOTS):][:items * S].reshape(items, S),
        link_seq=W[h(_abi.W_OFF_LINK_SEQ):][:links],
        link_info=W[h(_abi.W_OFF_LINK_INFO):][:links * _abi.LINK_INFO_WORDS].reshape(
            links, _abi.LINK_INFO_WORDS),
        link_tok=W[h(_abi.W_OFF_LINK_TOK):][:links * S].reshape(links, S),
        seq_qh=W[h(_abi.W_OFF_SEQ_QH):][:nseq + 1],
        qh_rh=W[h(_abi.W_OFF_QH_RH):][:qh],
        qh_pos=W[h(_abi.W_OFF_QH_POS):][:qh],
        seq_maxpos=W[h(_abi.W_OFF_SEQ_MAXPOS):][:nseq],
        listed=W[h(_abi.W_OFF_LISTED):][:h(_abi.W_LISTED)],
        seq_minpos=W[h(_abi.W_OFF_SEQ_MINPOS):][:nseq],
        seq_tok=W[h(_abi.W_OFF_SEQ_TOK):][:nseq + 1],
        tok_slot=W[h(_abi.W_OFF_TOK_SLOT):][:h(_abi.W_TOKENS)],
    )
    assert h(_abi.W_MAGIC) == _abi.PLAN_MAGIC and h(_abi.W_WORDS) == len(W)
    return t


def _brute_force(w, causal=True):
    """The pages' traversal, written out: returns (written slots, live slots,
    contributions {(slot, g, seq, token, row, head)})."""
    ps, heads, kv = w["page_size"], w["heads"], w["kv_heads"]
    group = heads // kv
    lens = w["seq_lens"].numpy()
    bt = w["block_table"].numpy()
    qs, qp = w["query_seq"].numpy(), w["query_pos"].numpy()
    links = {}
    for s, L in enumerate(lens):
        for lp in range((int(L) + ps - 1) // ps):
            links.setdefault(int(bt[s, lp]), []).append((s, lp))
    written, live, contrib = set(), set(), set()
    for page, lk in links.items():
        for off in range(ps):
            slot = page * ps + off
            written.add(slot)
            for s, lp in lk:
                token = lp * ps + off
                if token >= lens[s]:
                    continue
                live.add(slot)
                for r in range(len(qs)):           # rows in packed order
                    if qs[r] != s or (causal and token > qp[r]):
                        continue
                    for g in range(kv):
                        for h in range(g * group, (g + 1) * group):
                            contrib.add((slot, g, s, token, r, h))
    return written, live, contrib


def _from_plan(w, plan, causal=True):
    t = _tables(plan)
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    group = heads // kv
    written, live, contrib = set(), set(), set()
    for it in range(len(t["item_slots"])):
        ents = t["item_slots"][it]
        for e in ents:
            if e >= 0:
                written.add(int(e) >> 1)
                if e & 1:
                    live.add(int(e) >> 1)
        for li in range(t["item_links"][it], t["item_links"][it + 1]):
            s = int(t["link_seq"][li])
            toks = t["link_tok"][li]
            mn, mx, allv, rq0, rnqh, rminp, rmaxp, rseq = t["link_info"][li]
            valid = toks[toks >= 0]
            assert mn == valid.min() and mx == valid.max()
            assert allv == int((toks >= 0).all())
            q0, q1 = t["seq_qh"][s], t["seq_qh"][s + 1]
            # the record repeats the linked sequence's own facts
            assert (rseq, rq0, rnqh) == (s, q0, q1 - q0)
            assert (rminp, rmaxp) == (t["seq_minpos"][s], t["seq_maxpos"][s])
            for lane in range(_abi.PLAN_ITEM_SLOTS):
                tok = int(toks[lane])
                if tok < 0:
                    continue
                assert ents[lane] >= 0 and ents[lane] & 1
                slot = int(ents[lane]) >> 1
                for k in range(q0, q1):
                    pos = int(t["qh_pos"][k])
                    if causal and tok > pos:
                        continue
                    for g in range(kv):
                        rh = int(t["qh_rh"][k]) + g * group
                        contrib.add((slot, g, s, tok, rh // heads, rh % heads))
    return written, live, contrib, t


CASES = [
    dict(seed=1, nseq=4, len_lo=5, len_hi=60, q_per_seq=5, page_size=4, heads=4, kv_heads=2),
    dict(seed=2, nseq=3, len_lo=20, len_hi=70, q_per_seq=8, page_size=16, heads=4, kv_heads=1,
         share_prefix_pages=2, shuffle_rows=True),
    dict(seed=3, nseq=2, len_lo=3, len_hi=9, q_per_seq=3, page_size=1, heads=2, kv_heads=2,
         share_prefix_pages=2),
    dict(seed=4, nseq=3, len_lo=100, len_hi=300, q_per_seq=6, page_size=256, heads=6, kv_heads=2,
         shuffle_rows=True),
    dict(seed=5, nseq=4, len_lo=30, len_hi=50, q_per_seq=4, page_size=48, heads=3, kv_heads=3,
         share_prefix_pages=1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}-ps{c['page_size']}")
@pytest.mark.parametrize("causal", [True, False])
def test_plan_matches_brute_force_walk(case, causal):
    w = sdpa_inputs.paged_workload(D=8, dtype=torch.float32, **case)
    plan = _plan(w)
    bw, bl, bc = _brute_force(w, causal)
    pw, pl, pc, t = _from_plan(w, plan, causal)
    assert pw == bw            # the slots the backward writes
    assert pl == bl            # slots some link reaches (others store zero)
    assert pc == bc            # every contribution, exactly once as a set
    assert sorted(t["listed"].tolist()) == sorted({s // w["page_size"] for s in bw})
    # every listed slot belongs to exactly one item lane
    ents = t["item_slots"][t["item_slots"] >= 0] >> 1
    assert len(ents) == len(set(ents.tolist())) == len(bw)


def test_plan_rows_keep_packed_order():
    w = sdpa_inputs.paged_workload(seed=9, nseq=3, len_lo=10, len_hi=40, q_per_seq=7,
                                   page_size=8, heads=8, kv_heads=2, D=8, dtype=torch.float32,
                                   shuffle_rows=True)
    t = _tables(_plan(w))
    qs = w["query_seq"].numpy()
    G = 4
    for s in range(3):
        rh = t["qh_rh"][t["seq_qh"][s]:t["seq_qh"][s + 1]]
        rows = rh[::G] // 8
        assert np.array_equal(rows, np.where(qs == s)[0])          # original packed order
        assert np.array_equal(rh.reshape(-1, G) % 8, np.tile(np.arange(G), (len(rows), 1)))
        assert t["seq_maxpos"][s] == w["query_pos"].numpy()[qs == s].max()
        assert t["seq_minpos"][s] == w["query_pos"].numpy()[qs == s].min()


def _plan_eval(w, plan, stats, causal=True, scale=None):
    """dK / dV from the plan tables alone, float64, the kernel's reading of them."""
    t = _tables(plan)
    heads, kv, D = w["heads"], w["kv_heads"], w["D"]
    group = heads // kv
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    q = w["q"].double().numpy().reshape(-1, D)       # [(row, head), D]
    dy = w["dy"].double().numpy().reshape(-1, D)
    kp = w["k_pool"].double().numpy()
    vp = w["v_pool"].double().numpy()
    st = stats.reshape(-1, 3)
    dk = np.zeros_like(kp)
    dv = np.zeros_like(vp)
    for it in range(len(t["item_slots"])):
        ents = t["item_slots"][it]
        lanes = np.where((ents >= 0) & (ents & 1 == 1))[0]
        slots = ents[lanes] >> 1
        for g in range(kv):
            K, V = kp[slots, g], vp[slots, g]
            for li in range(t["item_links"][it], t["item_links"][it + 1]):
                s = t["link_seq"][li]
                tok = t["link_tok"][li][lanes]
                sl = slice(t["seq_qh"][s], t["seq_qh"][s + 1])
                rh = t["qh_rh"][sl] + g * group
                pos = t["qh_pos"][sl]
                Q, G = q[rh], dy[rh]
                m, l, dl = st[rh, 0], st[rh, 1], st[rh, 2]
                vis = (tok[None, :] >= 0) & (l[:, None] > 0)
                if causal:
                    vis &= tok[None, :] <= pos[:, None]
                with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
                    P = np.where(vis, np.exp(scale * (Q @ K.T) - m[:, None]) / l[:, None], 0.0)
                    dS = np.where(vis, P * ((G @ V.T) - dl[:, None]) * scale, 0.0)
                dk[slots, g] += dS.T @ Q
                dv[slots, g] += P.T @ G
    return dk, dv


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
def test_plan_evaluation_equals_oracle(case):
    w = sdpa_inputs.paged_workload(D=8, dtype=torch.float32, nan_unused=False, **case)
    plan = _plan(w)
    kw = dict(heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"])
    stats = oracle.paged_row_stats(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], **kw)
    dk_ref, dv_ref = oracle.paged_kv_bwd(w, w["q"], w["dy"], w["k_pool"], w["v_pool"], stats,
                                         np.zeros(w["k_pool"].shape), np.zeros(w["v_pool"].shape),
                                         **kw)
    dk, dv = _plan_eval(w, plan, stats)
    np.testing.assert_allclose(dk, dk_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_ref, rtol=0, atol=1e-12)


def test_plan_words_bound_and_errors():
    lib = _abi.load_library()
    w = sdpa_inputs.paged_workload(seed=3, nseq=2, len_lo=10, len_hi=20, q_per_seq=2, page_size=4,
                                   heads=2, kv_heads=1, D=8, dtype=torch.float32)
    plan = _plan(w)
    lens = w["seq_lens"].numpy().astype(np.int32)
    bound = lib.attn_bwd_paged_plan_words(2, lens.ctypes.data, w["block_table"].shape[1], 4, 2, 1,
                                          4, w["pool_pages"])
    assert bound >= len(plan.words)
    with pytest.raises(sb.AttnError, match="kv_heads"):
        sb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"], heads=3,
                      kv_heads=2, page_size=4, pool_pages=w["pool_pages"])
    bad = w["block_table"].clone()
    bad[0, 0] = w["pool_pages"]
    with pytest.raises(sb.AttnError, match="outside"):
        sb.paged_plan(w["seq_lens"], bad, w["query_seq"], w["query_pos"], heads=2, kv_heads=1,
                      page_size=4, pool_pages=w["pool_pages"])
    qs = w["query_seq"].clone()
    qs[0] = 7
    with pytest.raises(sb.AttnError, match="query_seq"):
        sb.paged_plan(w["seq_lens"], w["block_table"], qs, w["query_pos"], heads=2, kv_heads=1,
                      page_size=4, pool_pages=w["pool_pages"])
    long = w["seq_lens"].clone()
    long[1] = 10_000
    with pytest.raises(sb.AttnError):
        sb.paged_plan(long, w["block_table"], w["query_seq"], w["query_pos"], heads=2, kv_heads=1,
                      page_size=4, pool_pages=w["pool_pages"])


def test_empty_plan():
    plan = sb.paged_plan(np.zeros(0, np.int32), np.zeros((0, 1), np.int32), np.zeros(0, np.int32),
                         np.zeros(0, np.int32), heads=4, kv_heads=2, page_size=16, pool_pages=3)
    assert plan.items == 0 and len(plan.listed_pages()) == 0


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
def test_plan_token_slots(case):
    """Token t of sequence s sits at block_table[s][t / page_size] * page_size + t % page_size."""
    w = sdpa_inputs.paged_workload(D=8, dtype=torch.float32, **case)
    t = _tables(_plan(w))
    ps, bt = w["page_size"], w["block_table"].numpy()
    for s, L in enumerate(w["seq_lens"].tolist()):
        got = t["tok_slot"][t["seq_tok"][s]:t["seq_tok"][s + 1]]
        want = [bt[s, k // ps] * ps + k % ps for k in range(L)]
        assert got.tolist() == want


@pytest.mark.parametrize("lengths", [[5000, 1, 1024, 2048, 3000], [100, 0, 4096], [1025]])
def test_plan_query_pieces(lengths):
    """Split form of the query side: each query block's tokens [0, len) are cut,
    in order, into pieces of at most 1024 tokens starting at multiples of 1024
    (one empty piece for an empty sequence); the grid order lists every piece
    once, longest first, ties in piece order."""
    w = sdpa_inputs.paged_workload(seed=41, lengths=lengths, q_per_seq=0, page_size=16,
                                   heads=8, kv_heads=2, D=8, dtype=torch.float32)
    # rows: 70 per sequence (two query blocks of 128 qh rows with group 4 -> 280 qh rows)
    qs, qp = [], []
    for s, L in enumerate(lengths):
        for i in range(70):
            qs.append(s)
            qp.append(max(L - 70, 0) + i)
    w["query_seq"] = torch.tensor(qs, dtype=torch.int32)
    w["query_pos"] = torch.tensor(qp, dtype=torch.int32)
    plan = _plan(w)
    W = plan.words
    nblk, npc = int(W[_abi.W_QBLK]), int(W[_abi.W_QPIECES])
    qb = W[W[_abi.W_OFF_QBLK]:W[_abi.W_OFF_QBLK] + 2 * nblk].reshape(nblk, 2)
    pcs = W[W[_abi.W_OFF_QPIECE]:W[_abi.W_OFF_QPIECE] + 3 * npc].reshape(npc, 3)
    csr = W[W[_abi.W_OFF_QBLK_PIECE]:W[_abi.W_OFF_QBLK_PIECE] + nblk + 1]
    order = W[W[_abi.W_OFF_QPIECE_ORDER]:W[_abi.W_OFF_QPIECE_ORDER] + npc]
    T = _abi.PLAN_QPIECE_TOKENS
    assert csr[0] == 0 and csr[-1] == npc
    for b in range(nblk):
        L = lengths[qb[b, 0]]
        mine = pcs[csr[b]:csr[b + 1]]
        assert (mine[:, 0] == b).all()
        want = [(t, min(L, t + T)) for t in range(0, L, T)] or [(0, 0)]
        assert [tuple(x) for x in mine[:, 1:]] == want
    assert sorted(order.tolist()) == list(range(npc))
    ln = pcs[order, 2] - pcs[order, 1]
    assert (np.diff(ln) <= 0).all()
    for i in range(1, npc):  # stable: equal lengths keep piece order
        if ln[i] == ln[i - 1]:
            assert order[i] > order[i - 1]
