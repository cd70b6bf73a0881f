"""Benchmark of the paged attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Headline (``value``): causal prefill TFLOP/s on the Llama-3.2-1B attention
shape -- 2 sequences x 2048 tokens, 32 q heads, 8 KV heads, head_dim 64, bf16,
K/V in a 2 GiB pool of 65536 pages of 32768 B.  One step is the whole prefill
path: kv_scatter of all 4096 prompt tokens into their pages, then attn_prefill.
FLOPs follow the FlashAttention-2 explainer's convention (forward = 4 T^2 d H
per sequence, halved when causal).

Second object (``decode``): one decode step of 64 sequences with context
lengths uniform in [1, 2048] -- kv_scatter of the 64 newest tokens, then
attn_decode over every cached token -- as KV-read GB/s.  Eight replicas of the
cache on disjoint pages (over 1 GB in total) are cycled so a step never finds
the previous step's KV in the 256 MB last-level cache.

``roofline`` objects time the dominant kernel alone with HIP events on the
stream it runs on; ``cpu_baseline`` times the fp64 CPU oracle on the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_amd as pa  # noqa: E402
import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
DEV = torch.device("cuda")


def i32(x) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def device_pool(cache) -> torch.Tensor:
    fill = cache.page_fill if cache.page_fill < 0x8000 else cache.page_fill - 0x10000
    return torch.full((cache.pool_bytes // 2,), fill, dtype=torch.int16, device=DEV).view(torch.uint8)


def prefill_flops(B: int, T: int, Hq: int, d: int, causal: bool) -> float:
    f = 4.0 * T * T * d * Hq * B
    return f / 2 if causal else f


def time_launches(fn, n: int) -> float:
    """Mean device time (s) of one fn() call, from an event pair around each call."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in ev])) / 1e3


def timed_steps(step, steps: int, warmup: int) -> float:
    """Wall time (s) of `steps` steps after `warmup`, bracketed by device syncs."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


# ----------------------------------------------------------------- prefill

def bench_prefill(steps: int, warmup: int):
    case = W.llama_prefill()
    c = case.cache
    pool = device_pool(c)
    bt = i32(c.block_table)
    k = case.tokens.k.to(DEV)
    v = case.tokens.v.to(DEV)
    slots = i32(case.tokens.slot_ids)
    pos = i32(case.tokens.positions)
    q = case.q.to(DEV)
    lens = i32(case.seq_lens)
    sid = i32(case.slot_ids)
    O = torch.empty_like(q)
    L = torch.empty(case.B, case.Hq, case.T, dtype=torch.float32, device=DEV)

    def scatter():
        pa.kv_scatter(k, v, slots, pos, pool, bt, c.layer)

    def prefill():
        pa.attn_prefill(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, True, slot_ids=sid,
                        out=O, lse=L)

    def step(_):
        scatter()
        prefill()

    wall = timed_steps(step, steps, warmup)
    flops = prefill_flops(case.B, case.T, case.Hq, case.d, True)
    t_kernel = time_launches(prefill, max(steps, 20))
    t_scatter = time_launches(scatter, max(steps, 20))
    return dict(case=case, wall=wall, flops=flops, t_kernel=t_kernel, t_scatter=t_scatter)


# ------------------------------------------------------------------ decode

def decode_replicas(case, n: int):
    """Block tables placing the same contexts on n disjoint page sets."""
    bt0 = case.cache.block_table
    used = np.flatnonzero(bt0.reshape(-1) >= 0)
    n_used = len(used)
    perm = np.random.default_rng(1).permutation(case.cache.n_pages)
    tables = []
    for r in range(n):
        bt = np.full_like(bt0, -1).reshape(-1)
        bt[used] = perm[r * n_used:(r + 1) * n_used]
        tables.append(bt.reshape(bt0.shape))
    return tables


def bench_decode(steps: int, warmup: int, replicas: int = 8):
    case = W.llama_decode()
    c = case.cache
    pool = device_pool(c)
    tables = [i32(t) for t in decode_replicas(case, replicas)]
    ctx_k, ctx_v = case.context.k.to(DEV), case.context.v.to(DEV)
    ctx_s, ctx_p = i32(case.context.slot_ids), i32(case.context.positions)
    new_k, new_v = case.new_tokens.k.to(DEV), case.new_tokens.v.to(DEV)
    new_s, new_p = i32(case.new_tokens.slot_ids), i32(case.new_tokens.positions)
    for bt in tables:                                   # the cached context of every replica
        pa.kv_scatter(ctx_k, ctx_v, ctx_s, ctx_p, pool, bt, c.layer)
    q = case.q.to(DEV)
    lens = i32(case.ctx_lens)
    sid = i32(case.slot_ids)
    max_ctx = case.max_ctx
    ws = pa.decode_workspace(case.B, case.Hq, c.n_kv_heads, case.d, max_ctx, DEV)
    O = torch.empty_like(q)
    L = torch.empty(case.B, case.Hq, dtype=torch.float32, device=DEV)

    def scatter(r):
        pa.kv_scatter(new_k, new_v, new_s, new_p, pool, tables[r % replicas], c.layer)

    def decode(r):
        pa.attn_decode(q, pool, tables[r % replicas], c.layer, lens, c.n_kv_heads, case.scale,
                       max_ctx, slot_ids=sid, workspace=ws, out=O, lse=L)

    def step(i):
        scatter(i)
        decode(i)

    wall = timed_steps(step, steps, warmup)
    n_ctx = int(case.ctx_lens.sum())
    kv_bytes = n_ctx * c.n_kv_heads * case.d * 2 * 2
    io_bytes = q.numel() * 2 + O.numel() * 2 + L.numel() * 4 + int(np.ceil(case.ctx_lens / 16).sum()) * 4
    counter = iter(range(10**9))
    t_kernel = time_launches(lambda: decode(next(counter)), max(steps, 40))
    return dict(case=case, wall=wall, kv_bytes=kv_bytes, io_bytes=io_bytes, t_kernel=t_kernel,
                replicas=replicas, n_ctx=n_ctx)


# -------------------------------------------------------------- CPU oracle

def cpu_prefill_baseline(case):
    import oracle
    pool = oracle.pool_for(case)
    oracle.scatter_tokens(pool, case.cache, case.tokens)
    t0 = time.perf_counter()
    oracle.prefill_case(case, pool=pool)
    dt = time.perf_counter() - t0
    flops = prefill_flops(case.B, case.T, case.Hq, case.d, True)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole workload (2 x 2048 rows x 32 heads, fp64, {dt:.2f} s)"}


def cpu_decode_baseline(case):
    import oracle
    pool = oracle.pool_for(case)
    oracle.scatter_tokens(pool, case.cache, case.context)
    oracle.scatter_tokens(pool, case.cache, case.new_tokens)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_case(case, pool=pool)
        reps += 1
        if time.perf_counter() - t0 > 2.0:
            break
    dt = (time.perf_counter() - t0) / reps
    kv = int(case.ctx_lens.sum()) * case.cache.n_kv_heads * case.d * 4
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"the whole decode step, {reps} repeats ({dt:.3f} s each)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    pa.load()

    p = bench_prefill(args.steps, args.warmup)
    d = bench_decode(args.steps, args.warmup)

    case = p["case"]
    ms = p["wall"] / args.steps * 1e3
    value = p["flops"] / (p["wall"] / args.steps) / 1e12
    kern_tflops = p["flops"] / p["t_kernel"] / 1e12
    dcase = d["case"]
    d_ms = d["wall"] / args.steps * 1e3
    d_alg = d["kv_bytes"] + d["io_bytes"]
    d_kern = d_alg / d["t_kernel"] / 1e9

    out = {
        "metric": "causal prefill TFLOP/s (% bf16 MFMA peak); decode KV-read GB/s (% HBM peak)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "paged causal prefill, Llama-3.2-1B attention shape",
                   "batch": case.B, "seq_len": case.T, "q_heads": case.Hq,
                   "kv_heads": case.cache.n_kv_heads, "head_dim": case.d, "page_tokens": 16,
                   "pool_pages": case.cache.n_pages, "step": "kv_scatter(4096 tokens) + attn_prefill",
                   "flops_per_step": p["flops"], "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"kernel": "prefill_kernel<64,4,paged>", "bound": "mfma",
                     "achieved": round(kern_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_us": round(p["t_kernel"] * 1e6, 3)},
        "scatter_us": round(p["t_scatter"] * 1e6, 3),
        "decode": {
            "metric": "decode KV-read GB/s", "unit": "GB/s",
            "value": round(d["kv_bytes"] / (d["wall"] / args.steps) / 1e9, 2),
            "ms_per_step": round(d_ms, 5),
            "pct_of_hbm_peak": round(100 * d["kv_bytes"] / (d["wall"] / args.steps) / 1e9 / PEAK_HBM_GBS, 2),
            "config": {"workload": "paged decode step, 64 sequences, ctx ~ U[1, 2048]",
                       "batch": dcase.B, "ctx_tokens": d["n_ctx"], "kv_bytes": d["kv_bytes"],
                       "replicas": d["replicas"], "step": "kv_scatter(64 tokens) + attn_decode"},
            "roofline": {"kernel": "attn_decode (partial + combine)", "bound": "hbm",
                         "achieved": round(d_kern, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(d_kern / PEAK_HBM_GBS, 4), "traffic": None,
                         "avg_us": round(d["t_kernel"] * 1e6, 3), "alg_bytes": d_alg},
        },
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_prefill_baseline(case)
        out["decode"]["cpu_baseline"] = cpu_decode_baseline(dcase)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
