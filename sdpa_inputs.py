"""Seeded synthetic inputs for the attention-backward tests and benchmark.

This module only draws numbers and builds index tables; it holds none of the
attention arithmetic.  Both the GPU path and the CPU oracle are fed from it.

All draws use a torch CPU ``Generator`` seeded explicitly, values drawn as
float64 and then rounded (round-to-nearest-even) to the storage dtype, so the
oracle receives exactly the values the GPU receives.

The five workloads:
  1. fp32 [B1, S64, H2, D32], no mask, N(0,1).
  2. fp32 [B2, S512, H8, D64], causal; Q, K ~ 0.5 N(0,1); V, dY ~ N(0,1).
  3. bf16 [B4, S2048, H16, D128], N(0,1); sliding window w=256 (and plain causal).
  4. fp32 B2 H8 Sq128 Sk1024 D64 (queries are the last 128 positions):
     (a) per-batch key validity with the final UniformInt[0, 256] keys invalid,
     (b) additive fp32 bias [B, H, Sq, Sk] ~ N(0,1).
  5. paged grouped-query history: bf16, 32 query heads / 8 KV heads, D128,
     page 16, 16 sequences with lengths UniformInt[256, 4096], 64 queries per
     sequence at its last positions, pages scattered by a random permutation
     through a pool with 25% unused pages.
"""
from __future__ import annotations

import math

import torch

SEED_BASE = 1000


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(g, shape, dtype, mult=1.0):
    x = torch.randn(*shape, generator=g, dtype=torch.float64)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def dense_inputs(B, Sq, Sk, H, D, *, seed, dtype=torch.float32, qk_mult=1.0):
    """Q, dY: [B, Sq, H, D]; K, V: [B, Sk, H, D]; drawn in the order Q, K, V, dY."""
    g = _gen(seed)
    q = _randn(g, (B, Sq, H, D), dtype, qk_mult)
    k = _randn(g, (B, Sk, H, D), dtype, qk_mult)
    v = _randn(g, (B, Sk, H, D), dtype)
    dy = _randn(g, (B, Sq, H, D), dtype)
    return q, k, v, dy, g


def keypad_valid(g, B, Sk, max_invalid):
    """[B, Sk] float32 key validity: 1 for valid keys, 0 for the final n_b keys,
    n_b ~ UniformInt[0, max_invalid]."""
    n_inv = torch.randint(0, max_invalid + 1, (B,), generator=g)
    j = torch.arange(Sk)
    return (j[None, :] < (Sk - n_inv)[:, None]).to(torch.float32), n_inv


def bias_normal(g, B, H, Sq, Sk):
    return _randn(g, (B, H, Sq, Sk), torch.float32)


def config(k: int) -> dict:
    """Shapes and mask settings of workload k (1..5)."""
    if k == 1:
        return dict(B=1, H=2, Sq=64, Sk=64, D=32, dtype=torch.float32, mask="none")
    if k == 2:
        return dict(B=2, H=8, Sq=512, Sk=512, D=64, dtype=torch.float32, mask="causal",
                    qk_mult=0.5)
    if k == 3:
        return dict(B=4, H=16, Sq=2048, Sk=2048, D=128, dtype=torch.bfloat16,
                    mask="window", window=256)
    if k == 4:
        return dict(B=2, H=8, Sq=128, Sk=1024, D=64, dtype=torch.float32,
                    mask="keypad_or_bias", max_invalid=256)
    if k == 5:
        return dict(nseq=16, len_lo=256, len_hi=4096, q_per_seq=64, page_size=16,
                    unused_frac=0.25, heads=32, kv_heads=8, D=128, dtype=torch.bfloat16)
    raise ValueError(k)


def dense_config_inputs(k: int, seed=None):
    c = config(k)
    seed = SEED_BASE + k if seed is None else seed
    q, kk, v, dy, g = dense_inputs(c["B"], c["Sq"], c["Sk"], c["H"], c["D"], seed=seed,
                                   dtype=c["dtype"], qk_mult=c.get("qk_mult", 1.0))
    out = dict(cfg=c, q=q, k=kk, v=v, dy=dy)
    if k == 4:
        out["valid"], out["n_invalid"] = keypad_valid(g, c["B"], c["Sk"], c["max_invalid"])
        out["bias"] = bias_normal(g, c["B"], c["H"], c["Sq"], c["Sk"])
    return out


def hash_inputs(n, seed):
    """The deterministic generator of the rlx-cpu attention_bwd.rs unit test
    `all_matches_three_separate`: value_i = ((i * 2654435761 + seed) mod 1000) / 500 - 1."""
    i = torch.arange(n, dtype=torch.int64)
    return (((i * 2654435761 + seed) % 1000).to(torch.float64) / 500.0 - 1.0).to(torch.float32)


def paged_workload(*, seed, nseq=16, len_lo=256, len_hi=4096, q_per_seq=64, page_size=16,
                   unused_frac=0.25, heads=32, kv_heads=8, D=128, dtype=torch.bfloat16,
                   share_prefix_pages=0, shuffle_rows=False, nan_unused=True,
                   lengths=None, position_dim=0):
    """A paged KV pool and packed query rows.

    Draw order: lengths, page permutation, (row shuffle), Q, dY, K pool, V pool.
    Sequence s, logical page p maps to physical page block_table[s, p]; the first
    U = sum ceil(len_s / page_size) entries of a random permutation of the
    N = ceil(U / (1 - unused_frac)) pool pages are handed out in sequence-major
    order, the rest stay unused.  With ``share_prefix_pages`` = n > 0, every
    sequence after the first reuses the first n physical pages of sequence 0
    (a shared prefix), so those pages have several (sequence, logical page) links.
    Row r of sequence s sits at position len_s - q_per_seq + i.  Tail slots and
    unused pages of the K/V pools hold NaN when ``nan_unused``.
    With ``position_dim`` = P > 0 (the latent variant, where the K pool holds
    the latents) the draw continues with qp [nq, heads, P] and the position-key
    pool kp_pool [slots, kv_heads, P], NaN at the same slots.
    """
    g = _gen(seed)
    if lengths is None:
        lens = torch.randint(len_lo, len_hi + 1, (nseq,), generator=g)
    else:
        lens = torch.as_tensor(lengths, dtype=torch.int64)
        nseq = int(lens.numel())
    lens = torch.clamp(lens, min=q_per_seq) if q_per_seq > 0 else lens
    npages = [(int(L) + page_size - 1) // page_size for L in lens]
    share = [min(share_prefix_pages, npages[0], n) if s > 0 else 0
             for s, n in enumerate(npages)]
    used = sum(n - sh for n, sh in zip(npages, share))
    pool_pages = max(1, math.ceil(used / (1.0 - unused_frac)))
    perm = torch.randperm(pool_pages, generator=g)
    max_pages = max(npages) if npages else 1
    bt = torch.full((nseq, max(max_pages, 1)), -1, dtype=torch.int32)
    nxt = 0
    for s in range(nseq):
        for p in range(npages[s]):
            if p < share[s]:
                bt[s, p] = bt[0, p]
            else:
                bt[s, p] = int(perm[nxt])
                nxt += 1
    rows_seq, rows_pos = [], []
    for s in range(nseq):
        L = int(lens[s])
        for i in range(q_per_seq):
            rows_seq.append(s)
            rows_pos.append(L - q_per_seq + i)
    query_seq = torch.tensor(rows_seq, dtype=torch.int32)
    query_pos = torch.tensor(rows_pos, dtype=torch.int32)
    if shuffle_rows and len(rows_seq):
        order = torch.randperm(len(rows_seq), generator=g)
        query_seq, query_pos = query_seq[order], query_pos[order]
    nq = int(query_seq.numel())
    q = _randn(g, (nq, heads, D), dtype)
    dy = _randn(g, (nq, heads, D), dtype)
    k_pool = _randn(g, (pool_pages * page_size, kv_heads, D), dtype)
    v_pool = _randn(g, (pool_pages * page_size, kv_heads, D), dtype)
    live = torch.zeros(pool_pages * page_size, dtype=torch.bool)
    for s in range(nseq):
        for t in range(int(lens[s])):
            live[int(bt[s, t // page_size]) * page_size + t % page_size] = True
    if nan_unused:
        k_pool[~live] = float("nan")
        v_pool[~live] = float("nan")
    out = dict(seq_lens=lens.to(torch.int32), block_table=bt, query_seq=query_seq,
               query_pos=query_pos, q=q, dy=dy, k_pool=k_pool, v_pool=v_pool,
               live_slots=live, pool_pages=pool_pages, page_size=page_size,
               heads=heads, kv_heads=kv_heads, D=D, dtype=dtype)
    if position_dim > 0:
        out["qp"] = _randn(g, (nq, heads, position_dim), dtype)
        kp_pool = _randn(g, (pool_pages * page_size, kv_heads, position_dim), dtype)
        if nan_unused:
            kp_pool[~live] = float("nan")
        out["kp_pool"] = kp_pool
        out["P"] = position_dim
    return out
