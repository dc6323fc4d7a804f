#!/usr/bin/env python3
"""Benchmark of the dense attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mask causal|window]
    python bench.py --workload paged|paged_mla [--steps K] [--warmup W]

Workload: bf16 Q, K, V, dY of shape [B=4, S=2048, H=16, D=128] (N(0,1), seeded,
already resident in HBM), fp32 accumulation, bf16 dQ, dK, dV, causal mask.  One
step is one attn_bwd call through the C ABI on the current stream (for bf16:
the fused statistics + dQ pass, then the KV-block-major dK / dV pass).  The K
timed steps run back to back between two synchronisations; throughput counts
10 * B * H * Sq * Sk * D flops (the method's five contractions, 2 D flops each
per visible pair), halved for the causal mask; the window variant counts its
visible pairs.

Prints one JSON line.  Besides the contract fields it carries
  per_step     the same call timed one step at a time (HIP events around each
               call) over max(100, K) steps: median, min, p90; and again with a
               512 MiB device write between steps (no operand left in L2 or the
               256 MB Infinity Cache), median and min;
  kernels_ms   each kernel's average, from the stage entry points timed with
               events between the launches (they give attn_bwd's bits);
  roofline     the step against the bf16 MFMA peak: achieved = the method's
               counted flops over the sum of the kernels' times, so `frac` is
               the fraction of the peak the method's work reaches; `traffic` is
               the step's HBM bytes from stored rocprofv3 FETCH_SIZE /
               WRITE_SIZE measurements taken on the current kernel source, else
               null;
  issued_mfma  per kernel: the contractions it issues per visible pair (the
               dK / dV pass and the fused pass both recompute S and dP), its
               issued rate against the peak, and the SQ_VALU_MFMA_BUSY share
               measured on the current source (stored counters), else null;
  cpu_baseline the float64 CPU oracle on a bounded sample of the same workload:
               one thread on one (b, h) head, and 16 threads (one GPU's share of
               the host) on 16 heads; the host's core count and CPU model;
  from_forward the same step when a forward's log-sum-exp and output replace
               the statistics (attn_bwd_from_forward);
  window256    the same tensors under the sliding window w = 256 (the parity
               workload of this shape), counted over its visible pairs;
  paged        the paged grouped-query history backward (below), its dK / dV
               call against the HBM roofline and its query side;
  fp32_configs the fp32 dense workloads (configs 1, 2 and 4 with key padding
               or bias under the causal rule) through attn_bwd, against the
               fp32 MFMA peak.

--workload paged measures the paged grouped-query history backward alone
(ruDNN `history_backward`): bf16, 32 query / 8 KV heads, D 128, page 16, 16
sequences of UniformInt[256, 4096] tokens scattered through a pool with 25%
unused pages, 64 queries per sequence at its last positions, causal, supplied
fp32 row statistics; one step = one attn_bwd_paged call (plan built and
uploaded beforehand).  Its roofline is HBM: algorithmic bytes (K / V history
read once, dK / dV written over the listed pages, Q, dY and statistics read
once) over the kernel time.  The line also times the query side (statistics
and dQ on the GPU, as two calls and as one fused call; split form, and the
direct form beside it) and gives the whole chain's rate (fused query side plus
dK / dV) counted like the dense metric (10 D flops per visible triple).

--workload paged_mla measures the latent variant of the same kernel on the same
page tables (16 query heads on one latent KV head of width 128 plus a position
key of width 64; --latent-dim picks another latent width): TFLOP/s over the
visible triples (4 (D + P) + 4 D flops each) against the MFMA peak, since at
16 query heads per latent row the kernel sits far above the HBM ridge.

--no-extras keeps only the headline measurement (for profiler runs, whose
per-kernel averages then cover the headline's launches alone).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0
# Contractions each kernel issues per visible (query, key) pair, 2 D flops each.
CONTRACTIONS = {"row_stats": 2, "kv": 4, "dq": 3, "stats_dq": 4}
KERNEL_NAMES = {"row_stats": "k_row_stats", "kv": "k_kv_bwd", "dq": "k_dq_bwd",
                "stats_dq": "k_stats_dq",
                # the paged workload's 2648 (item, KV head) units outnumber the CUs,
                # so the library runs the persistent form; the latent variant has
                # only the one-workgroup-per-unit form
                "paged": "k_paged_kv_persist", "paged_mla": "k_paged_kv_bwd"}
# Files whose content decides a kernel's code (a stored traffic measurement is
# used only while their hash is unchanged).
KERNEL_SOURCES = ["scaled_dot_product_bwd_amd/csrc/dense_kernels.hip",
                  "scaled_dot_product_bwd_amd/csrc/device_common.hpp",
                  "scaled_dot_product_bwd_amd/csrc/kv_core.hpp",
                  "scaled_dot_product_bwd_amd/csrc/q_core.hpp",
                  "scaled_dot_product_bwd_amd/csrc/sd_core.hpp",
                  "scaled_dot_product_bwd_amd/build.py"]
PAGED_SOURCES = ["scaled_dot_product_bwd_amd/csrc/paged_kernels.hip",
                 "scaled_dot_product_bwd_amd/csrc/paged.hpp",
                 "scaled_dot_product_bwd_amd/csrc/device_common.hpp",
                 "scaled_dot_product_bwd_amd/csrc/kv_core.hpp",
                 "scaled_dot_product_bwd_amd/build.py"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(Sq, Sk, mask, window):
    """Visible (query, key) pairs of one head under the index rule."""
    off = max(Sk - Sq, 0)
    total = 0
    for i in range(Sq):
        a = off + i
        hi = min(a, Sk - 1)
        lo = max(a - window, 0) if mask == "window" else 0
        total += max(hi - lo + 1, 0)
    return total


def source_hash(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, tag="b4h16s2048d128_causal", sources=None):
    """Per-launch HBM bytes from profiles/traffic_<kernel>_<tag>.txt, if measured on
    this kernel source (key: value lines)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAMES[kernel]}_{tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != source_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


HOST_SHARE = 16  # host threads one GPU's jobs may use on the test machines


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo), or None."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(q, k, v, dy, mask, window):
    """The float64 C oracle (untuned: the full S x S definition per head, plain
    loops) on a bounded sample of the workload: 1 thread on 1 (b, h) head, then
    min(16, nproc) threads on as many heads (one thread per head).  `value` is
    the multi-thread rate in the metric's counted TFLOP/s."""
    import oracle
    import torch
    B, S, H, D = q.shape
    nproc = os.cpu_count() or 1
    threads = max(1, min(HOST_SHARE, nproc, B * H))
    code = 1 if mask == "causal" else 3
    pairs = [(b, h) for b in range(B) for h in range(H)]

    def run(nheads, nthreads):
        sub = [torch.stack([x[b, :, h, :] for b, h in pairs[:nheads]], dim=1).unsqueeze(0)
               for x in (q, k, v, dy)]
        t0 = time.perf_counter()
        oracle.attn_bwd(*sub, mask_kind=code, window=window, nthreads=nthreads)
        dt = time.perf_counter() - t0
        return counted_flops(1, nheads, S, S, D, mask, window) / dt / 1e12, dt

    v1, dt1 = run(1, 1)
    vn, dtn = run(threads, threads)
    return {"value": vn, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{threads} of {B * H} (b,h) heads of the same workload on {threads} threads "
                      f"(one head each), {dtn:.2f} s wall; untuned float64 C oracle (full S x S "
                      f"definition per head)",
            "single_thread": {"value": v1, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"1 (b,h) head, {dt1:.2f} s wall"},
            "nproc": nproc, "host_share_threads": HOST_SHARE, "cpu_model": cpu_model()}


def time_calls(fn, n, torch, between=None):
    """n calls of fn, each bracketed by its own pair of HIP events on the current
    stream; `between` (untimed) runs before each call.  Returns the times in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        if between is not None:
            between()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def dist(ms):
    xs = sorted(ms)
    n = len(xs)
    return {"n": n, "median_ms": round(xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2]), 5),
            "min_ms": round(xs[0], 5), "p90_ms": round(xs[min(n - 1, int(0.9 * n))], 5)}


def stored_mfma_busy(kernel, tag="b4h16s2048d128_causal"):
    """SQ_VALU_MFMA_BUSY share of `kernel` from profiles/counters_dense_kernels_<tag>.txt
    when measured on the current kernel source, else None."""
    import re
    path = os.path.join(ROOT, "profiles", f"counters_dense_kernels_{tag}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha: (\w+)", text)
    if not m or m.group(1) != source_hash():
        return None
    m = re.search(rf"^{re.escape(KERNEL_NAMES[kernel])} \| MFMA busy per SIMD ([0-9.]+)%", text, re.M)
    return float(m.group(1)) / 100.0 if m else None


def dense_bytes(B, H, Sq, Sk, D, es):
    """Algorithmic HBM bytes of one dense step: Q, dY read, K, V read, dQ, dK, dV
    written once each, the four statistics planes written once and read once."""
    return es * D * H * B * (3 * Sq + 4 * Sk) + 2 * 4 * 4 * B * H * Sq


def preheat(step, torch, seconds):
    """Untimed steps for a fixed wall time before the warmup steps.  Measured on
    this part: the first ~60 back-to-back steps of the dense workload run up to
    ~40% slower while the clocks ramp (652 us for steps 0-19, 470 us from step
    ~60 on, flat over 600 steps), so a few warmup steps alone time the ramp.
    Returns (steps run, seconds) for the JSON line."""
    import time as _t
    t0 = _t.perf_counter()
    n = 0
    while _t.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n, _t.perf_counter() - t0


def counted_flops(B, H, Sq, Sk, D, mask, window):
    if mask == "causal":
        return 10.0 * B * H * Sq * Sk * D / 2
    return 10.0 * D * B * H * visible_pairs(Sq, Sk, mask, window)


def paged_stats_torch(w, dev, scale):
    """Input synthesis for the paged workload: fp32 (max, denominator, delta) per
    (row, head), with plain torch float32 ops on the device (the statistics are
    an input of this backward, as on the pages)."""
    import torch
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    group = heads // kv
    q = w["q"].to(dev).float()
    dy = w["dy"].to(dev).float()
    kp = w["k_pool"].to(dev)
    vp = w["v_pool"].to(dev)
    stats = torch.zeros(q.shape[0], heads, 3, device=dev)
    qs, qp = w["query_seq"].to(dev), w["query_pos"].to(dev)
    for s, L in enumerate(w["seq_lens"].tolist()):
        t = torch.arange(L, device=dev)
        slots = w["block_table"][s].to(dev).long()[t // ps] * ps + t % ps
        rows = torch.nonzero(qs == s).flatten()
        K = kp[slots].float().repeat_interleave(group, dim=1).permute(1, 2, 0).contiguous()
        V = vp[slots].float().repeat_interleave(group, dim=1).permute(1, 2, 0).contiguous()
        Q = q[rows].permute(1, 0, 2).contiguous()           # [heads, r, D]
        G = dy[rows].permute(1, 0, 2).contiguous()
        sc = torch.bmm(Q, K) * scale                        # [heads, r, L]
        vis = t[None, :] <= qp[rows][:, None]
        sc = sc.masked_fill(~vis[None], float("-inf"))
        m = sc.amax(-1)
        e = torch.exp(sc - m[..., None])
        den = e.sum(-1)
        dp = torch.bmm(G, V)
        delta = (e / den[..., None] * dp).sum(-1)
        stats[rows] = torch.stack([m, den, delta], -1).permute(1, 0, 2)
    return stats


def paged_bytes(w, plan):
    """Algorithmic HBM bytes of one paged backward: K / V history read once,
    dK / dV written over every listed slot, Q, dY and the statistics read once."""
    es = 2 if str(w["dtype"]).endswith("bfloat16") else 4
    kvd = w["kv_heads"] * w["D"] * es
    hist = int(w["seq_lens"].sum()) * kvd * 2
    out = len(plan.listed_pages()) * w["page_size"] * kvd * 2
    nq, heads, D = w["q"].shape
    return hist + out + nq * heads * D * es * 2 + nq * heads * 3 * 4


def paged_flops(w):
    """Visible (row, head, token) triples x 8 D (four contractions)."""
    total = 0
    qs, qp = w["query_seq"].tolist(), w["query_pos"].tolist()
    lens = w["seq_lens"].tolist()
    for s, p in zip(qs, qp):
        total += min(p + 1, lens[s])
    return 8.0 * w["D"] * w["heads"] * total


def cpu_baseline_paged(w, nseq):
    import numpy as np
    import oracle
    sub = {k: v for k, v in w.items()}
    keep = [s for s in range(nseq)]
    sub["seq_lens"] = w["seq_lens"][keep]
    sub["block_table"] = w["block_table"][keep]
    rows = [r for r, s in enumerate(w["query_seq"].tolist()) if s in keep]
    for n in ("query_seq", "query_pos", "q", "dy"):
        sub[n] = w[n][rows]
    threads = max(1, min(os.cpu_count() or 1, 16))
    kw = dict(heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"])
    t0 = time.perf_counter()
    st = oracle.paged_row_stats(sub, sub["q"], sub["dy"], w["k_pool"], w["v_pool"],
                                nthreads=threads, **kw)
    t1 = time.perf_counter()
    oracle.paged_kv_bwd(sub, sub["q"], sub["dy"], w["k_pool"], w["v_pool"], st,
                        np.zeros(w["k_pool"].shape), np.zeros(w["v_pool"].shape),
                        nthreads=threads, **kw)
    dt = time.perf_counter() - t1
    flops = paged_flops(sub)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{nseq} of {len(w['seq_lens'])} sequences ({int(sub['seq_lens'].sum())} "
                      f"tokens) of the same workload, float64 C oracle dK/dV "
                      f"({t1 - t0:.2f} s of statistics not counted), {dt:.2f} s wall on "
                      f"{threads} threads"}


def paged_measure(args, torch, sdb, dev, cpu=True):
    """The paged dK / dV call on the config-5 workload (and its query side),
    timed with HIP events; returns the measurements as a dict."""
    import ctypes
    import sdpa_inputs
    log("bench: generating the paged workload")
    w = sdpa_inputs.paged_workload(seed=1005)
    D = w["D"]
    scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    plan = sdb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                          heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"],
                          pool_pages=w["pool_pages"], device=dev)
    stats = paged_stats_torch(w, dev, scale)
    q, dy, kp, vp = (w[n].to(dev) for n in ("q", "dy", "k_pool", "v_pool"))
    dk, dv = torch.zeros_like(kp), torch.zeros_like(vp)
    a = sdb.make_paged_args(q, dy, kp, vp, stats, plan, dk, dv, causal=True, scale=scale)
    lib = sdb.load_library()
    handle = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        rc = lib.attn_bwd_paged(ctypes.byref(a), handle)
        if rc != 0:
            raise RuntimeError(lib.attn_bwd_last_error().decode())

    ph_steps, ph_s = preheat(step, torch, args.preheat)
    log(f"bench: paged preheat {ph_steps} steps ({ph_s:.3f} s), warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    per = dist(time_calls(step, max(100, args.steps), torch))
    if not all(torch.isfinite(x[w["live_slots"].to(dev)]).all().item() for x in (dk, dv)):
        raise RuntimeError("non-finite gradients in the benchmark output")
    # The query side (statistics and dQ on the GPU: attn_bwd_paged_row_stats and
    # attn_bwd_paged_dq, and both in one call, attn_bwd_paged_stats_dq), timed
    # the same way; reported beside the dK / dV line.  Split form (each block's
    # tokens in pieces of <= 1024, merged; the default) and the direct form (one
    # workgroup per block).  The full chain is the fused call plus dK / dV.
    st_gpu = torch.empty_like(stats)
    dq = torch.empty_like(q)
    qws = sdb.paged_q_workspace(plan, D, dev)
    q_ms, q_direct_ms = {}, {}
    for split, dst in ((True, q_ms), (False, q_direct_ms)):
        a.q_workspace = qws.data_ptr() if split else None
        a.q_workspace_bytes = qws.numel() if split else 0
        for name, fn, outp in (("row_stats", lib.attn_bwd_paged_row_stats, st_gpu),
                               ("dq", lib.attn_bwd_paged_dq, dq)):
            def qstep():
                rc = fn(ctypes.byref(a), ctypes.c_void_p(outp.data_ptr()), handle)
                if rc != 0:
                    raise RuntimeError(lib.attn_bwd_last_error().decode())
            for _ in range(args.warmup):
                qstep()
            torch.cuda.synchronize()
            t0.record()
            for _ in range(args.steps):
                qstep()
            t1.record()
            torch.cuda.synchronize()
            dst[name] = round(t0.elapsed_time(t1) / args.steps, 4)
        # both in one call (attn_bwd_paged_stats_dq; with the workspace the
        # library picks the form, a.q_form = 0)
        def fstep():
            rc = lib.attn_bwd_paged_stats_dq(ctypes.byref(a), ctypes.c_void_p(st_gpu.data_ptr()),
                                             ctypes.c_void_p(dq.data_ptr()), handle)
            if rc != 0:
                raise RuntimeError(lib.attn_bwd_last_error().decode())
        for _ in range(args.warmup):
            fstep()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            fstep()
        t1.record()
        torch.cuda.synchronize()
        dst["stats_dq_fused"] = round(t0.elapsed_time(t1) / args.steps, 4)
    # the fused call's split form, forced (for the record)
    a.q_workspace, a.q_workspace_bytes, a.q_form = qws.data_ptr(), qws.numel(), 1
    for _ in range(args.warmup):
        fstep()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        fstep()
    t1.record()
    torch.cuda.synchronize()
    q_ms["stats_dq_fused_split_form"] = round(t0.elapsed_time(t1) / args.steps, 4)
    a.q_form = 0
    nbytes = paged_bytes(w, plan)
    flops = paged_flops(w)
    gbs = nbytes / (ms / 1e3) / 1e9
    tflops = flops / (ms / 1e3) / 1e12
    cpu_line = None
    if cpu and not args.no_cpu_baseline:
        log("bench: CPU oracle baseline on 2 sequences")
        cpu_line = cpu_baseline_paged(w, 2)
    wl = (f"paged_gqa_bwd nseq16 len[256,4096] heads32/8 D128 page16 q64/seq bf16 causal "
          f"(tokens {int(w['seq_lens'].sum())}, pool pages {w['pool_pages']})")
    return {
        "metric": "paged GQA history bwd (dK+dV) TFLOP/s & HBM GB/s",
        "value": round(tflops, 3), "unit": "TFLOP/s", "steps": args.steps,
        "warmup": args.warmup, "preheat": {"steps": ph_steps, "s": round(ph_s, 3)},
        "ms_per_step": round(ms, 5), "per_step": per,
        "config": {"workload": wl, "counted_flops": flops, "algorithmic_bytes": nbytes,
                   "items": plan.items},
        "pct_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS["bf16"], 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic("paged", "paged_config5", PAGED_SOURCES),
                     "kernel": KERNEL_NAMES["paged"], "kernel_ms": round(ms, 4),
                     "bytes_per_launch": nbytes},
        "query_side_ms": q_ms,
        "query_side_direct_ms": q_direct_ms,
        "full_chain_ms": round(ms + q_ms["stats_dq_fused"], 4),
        "full_chain_tflops": round(flops * 10.0 / 8.0 / ((ms + q_ms["stats_dq_fused"]) / 1e3) / 1e12, 3),
        "full_chain_separate_ms": round(ms + q_ms["row_stats"] + q_ms["dq"], 4),
        "cpu_baseline": cpu_line,
    }


def main_paged(args, torch, sdb, dev):
    m = paged_measure(args, torch, sdb, dev)
    line = {"metric": m.pop("metric"), "value": m.pop("value"), "unit": m.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": m.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    line.update(m)
    print(json.dumps(line), flush=True)


def paged_mla_stats_torch(w, dev, scale):
    """Input synthesis for the latent workload: fp32 (max, denominator, delta)
    per (row, head) with plain torch float32 ops on the device; the score is
    scale (q . c + qp . kp) and dP = dY . c (the latent c is key and value)."""
    import torch
    heads, kv, ps = w["heads"], w["kv_heads"], w["page_size"]
    group = heads // kv
    q, qp, dy = (w[n].to(dev).float() for n in ("q", "qp", "dy"))
    lat, kpp = w["k_pool"].to(dev), w["kp_pool"].to(dev)
    stats = torch.zeros(q.shape[0], heads, 3, device=dev)
    qs, qpos = w["query_seq"].to(dev), w["query_pos"].to(dev)
    for s, L in enumerate(w["seq_lens"].tolist()):
        t = torch.arange(L, device=dev)
        slots = w["block_table"][s].to(dev).long()[t // ps] * ps + t % ps
        rows = torch.nonzero(qs == s).flatten()
        C = lat[slots].float().repeat_interleave(group, dim=1).permute(1, 2, 0).contiguous()
        KP = kpp[slots].float().repeat_interleave(group, dim=1).permute(1, 2, 0).contiguous()
        sc = (torch.bmm(q[rows].permute(1, 0, 2).contiguous(), C)
              + torch.bmm(qp[rows].permute(1, 0, 2).contiguous(), KP)) * scale
        vis = t[None, :] <= qpos[rows][:, None]
        sc = sc.masked_fill(~vis[None], float("-inf"))
        m = sc.amax(-1)
        e = torch.exp(sc - m[..., None])
        den = e.sum(-1)
        dp = torch.bmm(dy[rows].permute(1, 0, 2).contiguous(), C)
        delta = (e / den[..., None] * dp).sum(-1)
        stats[rows] = torch.stack([m, den, delta], -1).permute(1, 0, 2)
    return stats


def paged_mla_counts(w, plan):
    """Latent workload: flops per visible (row, head, token) = 2 (D + P) for the
    score, 2 D for dP, 2 D for P^T dY and 2 (D + P) for dS^T [q | qp]; bytes =
    latent and position-key history read once, both gradients written over the
    listed slots, q, qp, dY and the statistics read once."""
    D, P = w["D"], w["P"]
    total = 0
    lens = w["seq_lens"].tolist()
    for s, p in zip(w["query_seq"].tolist(), w["query_pos"].tolist()):
        total += min(p + 1, lens[s])
    flops = (4.0 * (D + P) + 4.0 * D) * w["heads"] * total
    es = 2
    row = w["kv_heads"] * (D + P) * es
    nq, heads = w["q"].shape[:2]
    nbytes = (int(w["seq_lens"].sum()) * row + len(plan.listed_pages()) * w["page_size"] * row
              + nq * heads * (2 * D + P) * es + nq * heads * 3 * 4)
    return flops, nbytes


def main_paged_mla(args, torch, sdb, dev):
    import ctypes
    import numpy as np
    import sdpa_inputs
    log("bench: generating the latent paged workload")
    w = sdpa_inputs.paged_workload(seed=1005, heads=16, kv_heads=1, D=args.latent_dim,
                                   position_dim=64)
    D, P = w["D"], w["P"]
    scale = float(torch.tensor(1.0 / (D + P) ** 0.5, dtype=torch.float32))
    plan = sdb.paged_plan(w["seq_lens"], w["block_table"], w["query_seq"], w["query_pos"],
                          heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"],
                          pool_pages=w["pool_pages"], device=dev)
    stats = paged_mla_stats_torch(w, dev, scale)
    q, qp, dy, lat, kpp = (w[n].to(dev) for n in ("q", "qp", "dy", "k_pool", "kp_pool"))
    dl, dp = torch.zeros_like(lat), torch.zeros_like(kpp)
    a = sdb.make_paged_args(q, dy, lat, lat, stats, plan, dl, None, causal=True, scale=scale,
                            need=5)
    a.v_pool = None
    a.mla, a.position_dim = 1, P
    a.qp, a.kp_pool, a.dkp_pool = qp.data_ptr(), kpp.data_ptr(), dp.data_ptr()
    lib = sdb.load_library()

    def step():
        rc = lib.attn_bwd_paged(ctypes.byref(a), sdb._stream_handle(None))
        if rc != 0:
            raise RuntimeError(lib.attn_bwd_last_error().decode())

    ph_steps, ph_s = preheat(step, torch, args.preheat)
    log(f"bench: preheat {ph_steps} steps ({ph_s:.3f} s), warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    live = w["live_slots"].to(dev)
    if not all(torch.isfinite(x[live]).all().item() for x in (dl, dp)):
        raise RuntimeError("non-finite gradients in the benchmark output")
    flops, nbytes = paged_mla_counts(w, plan)
    tflops = flops / (ms / 1e3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("bench: CPU oracle baseline on 2 sequences")
        keep = [0, 1]
        sub = dict(w)
        sub["seq_lens"], sub["block_table"] = w["seq_lens"][keep], w["block_table"][keep]
        rows = [r for r, s_ in enumerate(w["query_seq"].tolist()) if s_ in keep]
        for n in ("query_seq", "query_pos", "q", "qp", "dy"):
            sub[n] = w[n][rows]
        kw = dict(heads=w["heads"], kv_heads=w["kv_heads"], page_size=w["page_size"])
        threads = max(1, min(os.cpu_count() or 1, 16))
        st = oracle.paged_mla_row_stats(sub, sub["q"], sub["qp"], sub["dy"], w["k_pool"],
                                        w["kp_pool"], scale=scale, nthreads=threads, **kw)
        c0 = time.perf_counter()
        oracle.paged_mla_kv_bwd(sub, sub["q"], sub["qp"], sub["dy"], w["k_pool"], w["kp_pool"],
                                st, np.zeros(w["k_pool"].shape), np.zeros(w["kp_pool"].shape),
                                scale=scale, nthreads=threads, **kw)
        dt = time.perf_counter() - c0
        sf, _ = paged_mla_counts(sub, plan)
        cpu = {"value": sf / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, w["kv_heads"]),
               "kind": "oracle",
               "sample": f"2 of {len(w['seq_lens'])} sequences ({int(sub['seq_lens'].sum())} "
                         f"tokens) of the same workload, float64 C oracle latent/position-key "
                         f"gradients, {dt:.2f} s wall (the oracle splits work by KV head: one "
                         f"thread here)"}
    wl = (f"paged_mla_bwd nseq16 len[256,4096] heads16/1 latent{D}+pos{P} page16 q64/seq bf16 "
          f"causal (tokens {int(w['seq_lens'].sum())}, pool pages {w['pool_pages']})")
    line = {
        "metric": "paged latent (MLA) history bwd (d latent + d pos-key) TFLOP/s",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "preheat": {"steps": ph_steps, "s": round(ph_s, 3)}, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "counted_flops": flops, "algorithmic_bytes": nbytes,
                   "items": plan.items},
        "pct_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS["bf16"], 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS["bf16"], 4),
                     "traffic": stored_traffic("paged_mla", "paged_mla", PAGED_SOURCES),
                     "kernel": KERNEL_NAMES["paged_mla"], "kernel_ms": round(ms, 4),
                     "flops_per_launch": flops, "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense", choices=["dense", "paged", "paged_mla"])
    ap.add_argument("--mask", default="causal", choices=["causal", "window"])
    ap.add_argument("--window", type=int, default=256)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline measurement (no scrubbed, from_forward, window or "
                         "paged parts): for profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--latent-dim", type=int, default=128, choices=[64, 128, 192, 256],
                    help="latent width of --workload paged_mla")
    ap.add_argument("--preheat", type=float, default=0.1,
                    help="seconds of untimed steps before the warmup steps (clock ramp)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the (b, h) "
              "heads are independent and would split across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sdpa_inputs
    import scaled_dot_product_bwd_amd as sdb

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return

    sdb.load_library()
    if args.workload == "paged":
        return main_paged(args, torch, sdb, dev)
    if args.workload == "paged_mla":
        return main_paged_mla(args, torch, sdb, dev)
    log("bench: generating inputs")
    d = sdpa_inputs.dense_config_inputs(3)
    qc, kc, vc, gc = d["q"], d["k"], d["v"], d["dy"]
    B, S, H, D = qc.shape
    window = args.window if args.mask == "window" else 0
    q, k, v, dy = (x.to(dev) for x in (qc, kc, vc, gc))
    head = dense_measure(args, torch, sdb, dev, (q, k, v, dy), args.mask, window, full=True)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline (1 thread on 1 head, then the host share)")
        cpu = cpu_baseline(qc, kc, vc, gc, args.mask, window)

    wl = f"sdpa_bwd B{B} H{H} S{S} D{D} bf16 " + (args.mask if args.mask == "causal"
                                                   else f"window{window}")
    line = {
        "metric": "attn-bwd TFLOP/s (dQ+dK+dV) & % MFMA peak, B4 H16 S2048 D128 bf16 causal",
        "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "preheat": head["preheat"], "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "B": B, "H": H, "Sq": S, "Sk": S, "D": D, "mask": args.mask,
                   "window": window if args.mask == "window" else None, "layout": "BSHD",
                   "entry": "attn_bwd", "counted_flops": head["counted_flops"]},
        "pct_mfma_peak": round(100.0 * head["tflops"] / PEAK_TFLOPS["bf16"], 3),
        "per_step": head["per_step"],
        "per_step_scrubbed": head["per_step_scrubbed"],
        "kernels_ms": head["kernels_ms"],
        "roofline": head["roofline"],
        "issued_mfma": head["issued_mfma"],
        "from_forward": head["from_forward"],
        "cpu_baseline": cpu,
    }
    if not args.no_extras and args.mask == "causal":
        log("bench: window-256 variant of the same tensors")
        wv = dense_measure(args, torch, sdb, dev, (q, k, v, dy), "window", args.window, full=False)
        line["window256"] = {k_: wv[k_] for k_ in ("ms_per_step", "tflops", "counted_flops",
                                                   "per_step", "kernels_ms", "roofline")}
        line["window256"]["pct_mfma_peak"] = round(100.0 * wv["tflops"] / PEAK_TFLOPS["bf16"], 3)
        del q, k, v, dy
        torch.cuda.empty_cache()
        pm = paged_measure(args, torch, sdb, dev, cpu=False)
        line["paged"] = {k_: pm[k_] for k_ in ("ms_per_step", "value", "unit", "per_step",
                                               "pct_mfma_peak", "roofline", "query_side_ms",
                                               "full_chain_ms", "full_chain_tflops", "config")}
        log("bench: fp32 dense workloads")
        line["fp32_configs"] = fp32_config_records(args, torch, sdb, dev)
    print(json.dumps(line), flush=True)


def fp32_config_records(args, torch, sdb, dev):
    """The fp32 dense workloads (configs 1, 2 and 4: the parity cases of the
    fp32 kernels k_row_stats, k_kv_bwd, k_dq_bwd), each timed through attn_bwd
    over >= 100 calls (per-call median): TFLOP/s counted over the pairs the
    index rule keeps (10 D flops each; key padding and bias hide or weight
    pairs inside that set, which the kernels compute like any other), against
    the fp32 MFMA peak.  Builder-side figures beside the bf16 headline."""
    import ctypes
    lib = sdb.load_library()
    recs = {}
    cases = [(1, "none", False), (2, "causal", False), (4, "keypad", True), (4, "bias", True)]
    for k, kind, causal in cases:
        d = sdpa_inputs_mod().dense_config_inputs(k)
        q, kk, v, dy = (d[n].to(dev) for n in ("q", "k", "v", "dy"))
        B, Sq, H, D = q.shape
        Sk = kk.shape[1]
        mask = None
        if kind == "keypad":
            mask = d["valid"].reshape(B, 1, 1, Sk).to(dev)
        elif kind == "bias":
            mask = d["bias"].to(dev)
        dq, dk, dv = (torch.empty_like(x) for x in (q, kk, v))
        # a workspace that allows the split form of the query-major passes
        # (the library uses it where the blocks would leave the GPU idle)
        ws = torch.empty(sdb.split_workspace_bytes(B, H, Sq, Sk, D), dtype=torch.uint8, device=dev)
        a = sdb.make_args(q, kk, v, dy, dq, dk, dv, mask_kind=kind, causal=causal, mask=mask,
                          workspace=ws)
        handle = sdb._stream_handle(None)

        def step():
            rc = lib.attn_bwd(ctypes.byref(a), handle)
            if rc != 0:
                raise RuntimeError(lib.attn_bwd_last_error().decode())
        for _ in range(max(args.warmup, 5)):
            step()
        per = dist(time_calls(step, max(100, args.steps), torch))
        pairs = visible_pairs(Sq, Sk, "causal", 0) if (kind == "causal" or causal) else Sq * Sk
        flops = 10.0 * D * B * H * pairs
        tf = flops / (per["median_ms"] / 1e3) / 1e12
        name = f"config{k}" + ("" if k != 4 else f"_{kind}_causal")
        recs[name] = {"workload": f"B{B} H{H} Sq{Sq} Sk{Sk} D{D} fp32 {kind}"
                                  + (" + causal" if causal else ""),
                      "per_step": per, "counted_flops": flops, "tflops": round(tf, 3),
                      "pct_fp32_mfma_peak": round(100.0 * tf / PEAK_TFLOPS["f32"], 3)}
        del q, kk, v, dy, dq, dk, dv, ws, mask
    torch.cuda.empty_cache()
    return recs


def sdpa_inputs_mod():
    import sdpa_inputs
    return sdpa_inputs


def dense_measure(args, torch, sdb, dev, tensors, mask, window, full):
    """One dense workload: the K-step timed region through attn_bwd, per-step
    times, per-kernel times from the stage entry points, the roofline and the
    issued-MFMA figures; with `full`, also the cache-scrubbed per-step times and
    the supplied-statistics (from_forward) step."""
    import ctypes
    q, k, v, dy = tensors
    B, S, H, D = q.shape
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    ws = torch.empty(sdb.workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
    a = sdb.make_args(q, k, v, dy, dq, dk, dv, mask_kind=mask, window=window, workspace=ws)
    lib = sdb.load_library()
    handle = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        rc = lib.attn_bwd(ctypes.byref(a), handle)
        if rc != 0:
            raise RuntimeError(lib.attn_bwd_last_error().decode())

    ph_steps, ph_s = preheat(step, torch, args.preheat)
    log(f"bench: {mask} preheat {ph_steps} steps ({ph_s:.3f} s), warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    # The timed region: K back-to-back attn_bwd calls between two synchronisations.
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    if not all(torch.isfinite(t).all().item() for t in (dq, dk, dv)):
        raise RuntimeError("non-finite gradients in the benchmark output")
    out = {"preheat": {"steps": ph_steps, "s": round(ph_s, 3)}, "ms_per_step": round(ms_step, 5)}
    out["per_step"] = dist(time_calls(step, max(100, args.steps), torch))
    if full and not args.no_extras:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fill = [0]

        def between():  # a 512 MiB write: no operand stays in L2 or the Infinity Cache
            fill[0] ^= 1
            scrub.fill_(fill[0])
        out["per_step_scrubbed"] = dist(time_calls(step, max(100, args.steps), torch, between))
        out["per_step_scrubbed"]["scrub_bytes"] = 512 << 20
        del scrub
    else:
        out["per_step_scrubbed"] = None

    # Per-kernel times: the bf16 sequence of attn_bwd through the stage entry
    # points (same kernels, same bits), events between the launches.
    stages = ["stats_dq", "kv"]
    n_k = max(30, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(n_k)]
    torch.cuda.synchronize()
    for e in evs:
        for i, st in enumerate(stages):
            e[i].record()
            sdb.attn_bwd_stage(st, a)
        e[len(stages)].record()
    torch.cuda.synchronize()
    per_kernel = {st: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / n_k
                  for i, st in enumerate(stages)}
    out["kernels_ms"] = {k_: round(v_, 4) for k_, v_ in per_kernel.items()}

    flops = counted_flops(B, H, S, S, D, mask, window)
    out["counted_flops"] = flops
    out["tflops"] = round(flops / (ms_step / 1e3) / 1e12, 3)
    kern_ms = sum(per_kernel.values())
    achieved = flops / (kern_ms / 1e3) / 1e12
    nbytes = dense_bytes(B, H, S, S, D, 2)
    ridge = PEAK_TFLOPS["bf16"] * 1e12 / (HBM_PEAK_GBS * 1e9)
    tag = "b4h16s2048d128_causal"
    traffic = None
    if mask == "causal":
        tr = [stored_traffic(st, tag) for st in stages]
        traffic = sum(tr) if all(t is not None for t in tr) else None
    # The bound follows the work's intensity against the ridge: MFMA-bound
    # workloads are measured in TFLOP/s, HBM-bound ones (the window band) in GB/s.
    if flops / nbytes > ridge:
        bound, ach, peak, unit = "mfma", achieved, PEAK_TFLOPS["bf16"], "TFLOP/s"
    else:
        bound, ach, peak, unit = "hbm", nbytes / (kern_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    out["roofline"] = {
        "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
        "frac": round(ach / peak, 4), "traffic": traffic,
        "mfma_frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
        "kernel": "attn_bwd step: " + " + ".join(KERNEL_NAMES[st] for st in stages),
        "kernel_ms": round(kern_ms, 4), "flops_per_launch": flops,
        "work": "10 D flops per visible (query, key) pair: the method's five contractions, "
                "each counted once per step",
        "algorithmic_bytes": nbytes, "intensity_flop_per_byte": round(flops / nbytes, 1),
        "ridge_flop_per_byte": round(ridge, 1)}
    pairs = flops / (10.0 * D)
    issued = {}
    for st in stages:
        f_ = 2.0 * D * CONTRACTIONS[st] * pairs
        t_ = f_ / (per_kernel[st] / 1e3) / 1e12
        issued[KERNEL_NAMES[st]] = {
            "ms": round(per_kernel[st], 4), "contractions_per_pair": CONTRACTIONS[st],
            "issued_tflops": round(t_, 2), "frac_of_peak": round(t_ / PEAK_TFLOPS["bf16"], 4),
            "counter_mfma_busy": stored_mfma_busy(st, tag) if mask == "causal" else None}
    out["issued_mfma"] = issued

    out["from_forward"] = None
    if full and not args.no_extras:
        # The same backward from a forward's saved statistics (attn_bwd_from_forward:
        # log-sum-exp and O replace the statistics pass).  Timing only: lse comes
        # from this run's statistics and O is a stand-in tensor of the right shape
        # (the kernels' cost does not depend on the values).
        m_ws, l_ws, _ = sdb.row_stats_views(ws, B, H, S)
        lse = (m_ws + torch.log(l_ws)).contiguous()
        o_stand = dy.clone()
        ost = (ctypes.c_int64 * 3)(*o_stand.stride()[:3])
        dq2, dk2, dv2 = (torch.empty_like(x) for x in (q, k, v))
        ws2 = torch.empty_like(ws)
        a2 = sdb.make_args(q, k, v, dy, dq2, dk2, dv2, mask_kind=mask, window=window, workspace=ws2)

        def fstep():
            rc = lib.attn_bwd_from_forward(ctypes.byref(a2), ctypes.c_void_p(lse.data_ptr()),
                                           ctypes.c_void_p(o_stand.data_ptr()), ost, handle)
            if rc != 0:
                raise RuntimeError(lib.attn_bwd_last_error().decode())
        preheat(fstep, torch, args.preheat)  # the clocks drop while the host prepares this segment
        for _ in range(args.warmup):
            fstep()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            fstep()
        t1.record()
        torch.cuda.synchronize()
        ff_ms = t0.elapsed_time(t1) / args.steps
        out["from_forward"] = {"ms_per_step": round(ff_ms, 5),
                               "tflops": round(flops / (ff_ms / 1e3) / 1e12, 3)}
    return out


if __name__ == "__main__":
    main()
