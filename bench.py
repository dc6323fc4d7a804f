#!/usr/bin/env python3
"""Benchmark of the dense attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mask causal|window]

Workload: bf16 Q, K, V, dY of shape [B=4, S=2048, H=16, D=128] (N(0,1), seeded,
already resident in HBM), fp32 accumulation, bf16 dQ, dK, dV, causal mask.  One
step is the whole backward: row statistics, the KV-block-major dK / dV kernel and
the query-block-major dQ kernel, each launched through the C ABI on the current
stream.  Throughput counts 10 * B * H * Sq * Sk * D flops (five contractions),
halved for the causal mask; the window variant counts its visible pairs.

Prints one JSON line.  Besides the contract fields it carries
  roofline     for the dominant kernel: algorithmic flops per launch over its
               average launch time (HIP events on the launch stream), against
               the MI355X dense bf16 MFMA peak; `traffic` comes from a stored
               rocprofv3 FETCH_SIZE / WRITE_SIZE measurement when it was taken
               on the current kernel source, else null;
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload.
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
CONTRACTIONS = {"row_stats": 2, "kv": 4, "dq": 3}
KERNEL_NAMES = {"row_stats": "k_row_stats", "kv": "k_kv_bwd", "dq": "k_dq_bwd"}
KERNEL_SOURCES = ["scaled_dot_product_bwd_amd/csrc/dense_kernels.hip",
                  "scaled_dot_product_bwd_amd/csrc/device_common.hpp"]


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


def source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """Per-launch HBM bytes from profiles/traffic_<kernel>_*.txt, if measured on
    this kernel source (key: value lines)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAMES[kernel]}_b4h16s2048d128_causal.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(q, k, v, dy, mask, window, nheads):
    import oracle
    B, S, H, D = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)][:nheads]
    import torch
    sub = [torch.stack([x[b, :, h, :] for b, h in pairs], dim=1).unsqueeze(0) for x in (q, k, v, dy)]
    threads = max(1, min(len(pairs), os.cpu_count() or 1, 16))
    code = 1 if mask == "causal" else 3
    t0 = time.perf_counter()
    oracle.attn_bwd(*sub, mask_kind=code, window=window, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = counted_flops(1, len(pairs), S, S, D, mask, window)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(pairs)} of {B * H} (b,h) heads of the same workload, float64 C "
                      f"oracle, {dt:.2f} s wall on {threads} threads"}


def counted_flops(B, H, Sq, Sk, D, mask, window):
    if mask == "causal":
        return 10.0 * B * H * Sq * Sk * D / 2
    return 10.0 * D * B * H * visible_pairs(Sq, Sk, mask, window)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mask", default="causal", choices=["causal", "window"])
    ap.add_argument("--window", type=int, default=256)
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="(b,h) heads the CPU oracle baseline processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the (b, h) heads are independent; see the design notes on sharding). "
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
    log("bench: generating inputs")
    d = sdpa_inputs.dense_config_inputs(3)
    qc, kc, vc, gc = d["q"], d["k"], d["v"], d["dy"]
    B, S, H, D = qc.shape
    window = args.window if args.mask == "window" else 0
    q, k, v, dy = (x.to(dev) for x in (qc, kc, vc, gc))
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    ws = torch.empty(sdb.workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
    a = sdb.make_args(q, k, v, dy, dq, dk, dv, mask_kind=args.mask, window=window, workspace=ws)
    stages = ["row_stats", "kv", "dq"]

    def step(ev=None):
        for i, st in enumerate(stages):
            if ev is not None:
                ev[i].record()
            sdb.attn_bwd_stage(st, a)
        if ev is not None:
            ev[len(stages)].record()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per_kernel = {st: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                  for i, st in enumerate(stages)}
    if not all(torch.isfinite(t).all().item() for t in (dq, dk, dv)):
        raise RuntimeError("non-finite gradients in the benchmark output")

    flops = counted_flops(B, H, S, S, D, args.mask, window)
    value = flops / (ms_step / 1e3) / 1e12
    pairs_step = flops / (10.0 * D)  # visible pairs as counted
    dom = max(per_kernel, key=per_kernel.get)
    dom_flops = 2.0 * D * CONTRACTIONS[dom] * pairs_step
    achieved = dom_flops / (per_kernel[dom] / 1e3) / 1e12
    traffic = stored_traffic(dom) if args.mask == "causal" else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                "traffic": traffic, "kernel": KERNEL_NAMES[dom],
                "kernel_ms": round(per_kernel[dom], 4),
                "flops_per_launch": dom_flops}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle baseline on {args.cpu_heads} heads")
        cpu = cpu_baseline(qc, kc, vc, gc, args.mask, window, args.cpu_heads)

    wl = f"sdpa_bwd B{B} H{H} S{S} D{D} bf16 " + (args.mask if args.mask == "causal"
                                                   else f"window{window}")
    line = {
        "metric": "attn-bwd TFLOP/s (dQ+dK+dV) & % MFMA peak, B4 H16 S2048 D128 bf16 causal",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "B": B, "H": H, "Sq": S, "Sk": S, "D": D, "mask": args.mask,
                   "window": window if args.mask == "window" else None, "layout": "BSHD",
                   "counted_flops": flops},
        "pct_mfma_peak": round(100.0 * value / PEAK_TFLOPS["bf16"], 3),
        "kernels_ms": {k_: round(v_, 4) for k_, v_ in per_kernel.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
