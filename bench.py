"""Benchmark of the paged attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--sustain S]

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
import hashlib
import re
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
SUSTAIN_S = 5.0                # seconds of back-to-back steps after the timed ones (--sustain)
DEV = torch.device("cuda")


def i32(x) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def device_pool(cache) -> torch.Tensor:
    fill = cache.page_fill if cache.page_fill < 0x8000 else cache.page_fill - 0x10000
    return torch.full((cache.pool_bytes // 2,), fill, dtype=torch.int16, device=DEV).view(torch.uint8)


def prefill_flops(B: int, T: int, Hq: int, d: int, causal: bool) -> float:
    f = 4.0 * T * T * d * Hq * B
    return f / 2 if causal else f


def capture(fn, reps: int = 1) -> torch.cuda.CUDAGraph:
    """A HIP graph holding `reps` back-to-back calls of fn (its kernels only)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm the path once outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def warm(g, seconds: float) -> None:
    """Replay graph g until `seconds` have passed.  Under a fresh load the GPU's
    clocks take about 0.1 s to ramp up (the Llama prefill kernel runs ~52 us in
    the first launches and ~42 us once the GPU is busy), so every measurement
    here is taken after such a warm-up: the steady state is what is reported."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()


def kernel_time(fn, reps: int = 20, trials: int = 5, warm_s: float = 0.1) -> float:
    """Average device time (s) of one call of fn: a graph of `reps` back-to-back
    calls is replayed `trials` times between two HIP events on the launching
    stream (after `warm_s` seconds of untimed replays); total time / (reps * trials)."""
    g = capture(fn, reps)
    warm(g, warm_s)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(trials):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / (reps * trials)


def launch_spread(fns, n: int = 50, warmup: int = 10) -> dict:
    """Median, p10 and p90 (us) of single launches, each between two HIP
    events on the launching stream, after `warmup` untimed ones; launch i runs
    fns[i % len(fns)].  A single-launch time also holds the gap between the
    event and the kernel (about a microsecond), which the graph averages of
    kernel_time do not."""
    warm(capture(lambda: [fn() for fn in fns]), 0.1)
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (s, e) in enumerate(ev):
        s.record()
        fns[i % len(fns)]()
        e.record()
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])
    return {"n": n, "median_us": round(float(np.median(t)), 2),
            "p10_us": round(float(np.percentile(t, 10)), 2), "p90_us": round(float(np.percentile(t, 90)), 2)}


def sustained(step_fns, seconds: float, per_graph: int = 8) -> dict:
    """The same steps replayed back to back for about `seconds` (graphs of
    `per_graph` steps, one device sync every 16 graphs): the steady-state time
    per step, beside the exactly-K-step timing, and a GPU busy long enough for
    an outside sampler to see."""
    n = len(step_fns)
    per_graph = max(n, per_graph - per_graph % n)
    g = capture(lambda: [step_fns[j % n]() for j in range(per_graph)])
    warm(g, 0.1)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            g.replay()
        torch.cuda.synchronize()
        done += 16 * per_graph
    dt = time.perf_counter() - t0
    return {"seconds": round(dt, 2), "steps": done, "ms_per_step": round(dt / done * 1e3, 5)}


def timed_steps(step_fns, steps: int, warmup: int, per_graph: int = 8) -> float:
    """Wall time (s) of exactly `steps` steps after 0.2 s of untimed replays
    (the clocks' ramp, see warm) and `warmup` steps, bracketed by device syncs.  Step i runs step_fns[i % n]; the steps are replayed from HIP graphs
    of `per_graph` consecutive steps (a multiple of n) plus one graph of the
    remainder, so the host launches one graph per `per_graph` steps."""
    n = len(step_fns)
    per_graph = max(n, per_graph - per_graph % n)

    def steps_graph(count: int):
        return capture(lambda: [step_fns[j % n]() for j in range(count)])

    full = steps_graph(per_graph)
    rem = steps % per_graph
    tail = steps_graph(rem) if rem else None
    warm(full, 0.2)   # clocks up before the warm-up steps proper
    for _ in range(-(-warmup // per_graph)):
        full.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // per_graph):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def source_digest(*names: str) -> str:
    """Digest of the code of the named sources: comments and runs of white
    space are dropped first, so that an edit of a comment leaves it (and the
    traffic measured on that code) unchanged."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# HBM traffic per launch measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (separate runs), scaled by the factor a plain copy kernel of
# known size reads on the same counters; valid only for the kernel source it
# was taken on (digest of the code of the .hip files, comments excluded),
# null otherwise.
TRAFFIC = {
    # kernel: (source digest, fetched bytes, written bytes)
    "prefill": ("f6b15280df2341e4", 25386829, 17301504),
    "decode": ("8d098f650bae1593", 152917154, 272998),
}


def traffic_of(kernel: str, digest: str):
    t = TRAFFIC.get(kernel)
    if not t or t[0] != digest:
        return None
    return t[1] + t[2]


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

    def step():
        scatter()
        prefill()

    # eager reference result, then the graph of one step must reproduce it
    step()
    torch.cuda.synchronize()
    O_ref, L_ref = O.clone(), L.clone()
    wall = timed_steps([step], steps, warmup)
    assert torch.equal(O, O_ref) and torch.equal(L, L_ref), "graph replay differs from eager"
    sus = sustained([step], SUSTAIN_S) if SUSTAIN_S > 0 else None
    flops = prefill_flops(case.B, case.T, case.Hq, case.d, True)
    alg_bytes = (q.numel() + O.numel()) * 2 + L.numel() * 4 + 2 * k.numel() * 2
    t_kernel = kernel_time(prefill)
    # the same step in one launch: attn_prefill_append writes the prompt's K/V
    # to the pages and attends to the rows of its inputs
    kd = k.view(case.B, case.T, c.n_kv_heads, case.d)
    vd = v.view(case.B, case.T, c.n_kv_heads, case.d)
    O2, L2 = torch.empty_like(O), torch.empty_like(L)

    def append_step():
        pa.attn_prefill_append(q, kd, vd, pool, bt, c.layer, lens, case.scale, True, slot_ids=sid,
                               out=O2, lse=L2)

    append_step()
    torch.cuda.synchronize()
    assert (O2.float() - O_ref.float()).abs().max().item() <= 2e-2 and (L2 - L_ref).abs().max().item() <= 1e-3
    wall_append = timed_steps([append_step], steps, warmup)
    return dict(case=case, wall=wall, flops=flops, t_kernel=t_kernel, clock_ghz=sustained_clock(), sustained=sus,
                t_scatter=kernel_time(scatter), alg_bytes=alg_bytes, spread=launch_spread([prefill]),
                wall_append=wall_append)


RATED_CLOCK_GHZ = 2.4          # the clock the 2.5 PFLOP/s bf16 figure is rated at


def sustained_clock() -> float:
    """Median shader clock (GHz) over 4096 waves that keep every SIMD issuing
    bf16 matrix products for about a millisecond (pa_clock_probe)."""
    pa.clock_probe(4096, 2000)          # untimed: raise the clock from idle
    ghz = pa.clock_probe(4096, 20000).cpu()
    return float(ghz.median())


# ------------------------------------------------------------------ decode

def decode_path_note(B: int, Hq: int, Hkv: int, d: int, max_ctx: int) -> str:
    """Which attn_decode kernel serves this shape, for the sweep's notes."""
    if pa.decode_whole_pages(B, Hq, Hkv, d, max_ctx):
        return "whole-page kernel (one workgroup per CU, equal page shares) + merge kernel"
    n = pa.decode_splits(B, Hq, Hkv, d, max_ctx)
    return "per-head kernel" + (f", {n} workgroup splits per context + combine kernel" if n > 1 else "")


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
        pa.kv_scatter(new_k, new_v, new_s, new_p, pool, tables[r], c.layer)

    def decode(r):
        pa.attn_decode(q, pool, tables[r], c.layer, lens, c.n_kv_heads, case.scale,
                       max_ctx, slot_ids=sid, workspace=ws, out=O, lse=L)

    def step(r):
        scatter(r)
        decode(r)

    step(0)
    torch.cuda.synchronize()
    O_ref, L_ref = O.clone(), L.clone()
    wall = timed_steps([lambda r=r: step(r) for r in range(replicas)], steps, warmup)
    assert torch.equal(O, O_ref) and torch.equal(L, L_ref), "graph replay differs from eager"
    sus = sustained([lambda r=r: step(r) for r in range(replicas)], SUSTAIN_S) if SUSTAIN_S > 0 else None
    n_ctx = int(case.ctx_lens.sum())
    kv_bytes = n_ctx * c.n_kv_heads * case.d * 2 * 2
    io_bytes = q.numel() * 2 + O.numel() * 2 + L.numel() * 4 + int(np.ceil(case.ctx_lens / 16).sum()) * 4
    # one launch per replica in turn: the KV of a launch is never the previous one's
    t_kernel = kernel_time(lambda: [decode(r) for r in range(replicas)], reps=4) / replicas
    # whole pages touched: ceil(ctx/16) pages of 16 tokens x all kv heads x (K, V)
    page_bytes = int(np.ceil(case.ctx_lens / 16).sum()) * 16 * c.n_kv_heads * case.d * 2 * 2
    spread = launch_spread([lambda r=r: decode(r) for r in range(replicas)])
    # the same step in one launch: attn_decode_append writes the 64 new tokens
    # and attends to them with the cached context
    O2, L2 = torch.empty_like(O), torch.empty_like(L)

    def append_step(r):
        pa.attn_decode_append(q, new_k, new_v, pool, tables[r], c.layer, lens, c.n_kv_heads, case.scale,
                              max_ctx, slot_ids=sid, workspace=ws, out=O2, lse=L2)

    append_step(0)
    torch.cuda.synchronize()
    assert (O2.float() - O_ref.float()).abs().max().item() <= 2e-2 and (L2 - L_ref).abs().max().item() <= 1e-3
    wall_append = timed_steps([lambda r=r: append_step(r) for r in range(replicas)], steps, warmup)
    return dict(case=case, wall=wall, kv_bytes=kv_bytes, io_bytes=io_bytes, t_kernel=t_kernel, sustained=sus,
                replicas=replicas, n_ctx=n_ctx, page_bytes=page_bytes, spread=spread, wall_append=wall_append)


# -------------------------------------------------------------- CPU oracle

def host_info() -> dict:
    """Host CPU facts for the oracle timings: model, logical CPUs, CPUs this
    process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def _repeat(fn, min_s: float):
    """Seconds per call of fn, called until min_s have passed (at least once)."""
    reps, t0 = 0, time.perf_counter()
    while reps < 1 or time.perf_counter() - t0 < min_s:
        fn()
        reps += 1
    return (time.perf_counter() - t0) / reps, reps


def spread_rows(B: int, T: int, per_seq: int, seqs=None) -> np.ndarray:
    """(b, t) rows spread evenly over the positions of sequences `seqs` (all by
    default): a sample whose causal cost is that of the whole in proportion."""
    ts = ((np.arange(per_seq) + 0.5) * T / per_seq).astype(np.int64)
    seqs = range(B) if seqs is None else seqs
    return np.array([(b, t) for b in seqs for t in ts], np.int32)


def row_flops(rows: np.ndarray, T: int, Hq: int, d: int, causal: bool, offset=None) -> float:
    """FLOPs of the given rows: 4 d Hq per visible (query, key) pair."""
    t = rows[:, 1].astype(np.int64)
    keys = (t + 1 + (0 if offset is None else offset[rows[:, 0]])) if causal else np.full_like(t, T)
    return 4.0 * d * Hq * float(keys.sum())


def _one_thread(fn):
    import oracle
    n = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        return fn()
    finally:
        oracle.set_num_threads(n)


def cpu_prefill_baseline(case):
    """The fp64 oracle on the Llama prefill: the whole workload on every thread,
    and an evenly spread row sample on one thread (its own FLOPs / its time)."""
    import oracle
    pool = oracle.pool_for(case)
    oracle.scatter_tokens(pool, case.cache, case.tokens)
    dt, reps = _repeat(lambda: oracle.prefill_case(case, pool=pool), 6.0)
    flops = prefill_flops(case.B, case.T, case.Hq, case.d, True)
    rows = spread_rows(case.B, case.T, 32)
    rf = row_flops(rows, case.T, case.Hq, case.d, True)
    dt1, reps1 = _one_thread(lambda: _repeat(lambda: oracle.prefill_case(case, rows=rows, pool=pool), 4.0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole workload (2 x 2048 rows x 32 heads, fp64), {reps} repeats of {dt:.2f} s",
            "one_thread": {"value": round(rf / dt1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                           "sample": f"{len(rows)} rows spread evenly over both sequences' positions "
                                     f"({rf / flops * 100:.2f}% of the FLOPs), {reps1} repeats of {dt1:.3f} s",
                           "whole_workload_s_extrapolated": round(flops * dt1 / rf, 2)},
            "host": host_info()}


def cpu_decode_baseline(case):
    """The fp64 oracle on the decode step: the whole step on every thread, and
    8 of the 64 sequences (every 8th by length) on one thread, as KV GB/s."""
    import oracle
    pool = oracle.pool_for(case)
    oracle.scatter_tokens(pool, case.cache, case.context)
    oracle.scatter_tokens(pool, case.cache, case.new_tokens)
    dt, reps = _repeat(lambda: oracle.decode_case(case, pool=pool), 4.0)
    per_tok = case.cache.n_kv_heads * case.d * 4
    kv = int(case.ctx_lens.sum()) * per_tok
    c = case.cache
    pick = np.argsort(case.ctx_lens, kind="stable")[4::8]
    sub = dict(q=case.q[torch.as_tensor(pick)], slot_ids=np.asarray(case.slot_ids)[pick], ctx=np.asarray(case.ctx_lens)[pick])
    kv1 = int(sub["ctx"].sum()) * per_tok

    def sample():
        oracle.attn_decode(sub["q"], pool, c.n_pages, c.block_table, c.layer, sub["slot_ids"], sub["ctx"],
                           c.n_kv_heads, case.scale)

    dt1, reps1 = _one_thread(lambda: _repeat(sample, 3.0))
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"the whole decode step, {reps} repeats ({dt:.3f} s each)",
            "one_thread": {"value": round(kv1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"8 of the 64 sequences (every 8th by context length, "
                                     f"{int(sub['ctx'].sum())} of {int(case.ctx_lens.sum())} tokens), "
                                     f"{reps1} repeats of {dt1:.3f} s",
                           "whole_step_s_extrapolated": round(kv * dt1 / kv1, 3)},
            "host": host_info()}


COPY_BYTES = 256 << 20


def kernels_only(n: int) -> None:
    """For hardware-counter runs: launch a plain copy of COPY_BYTES (the
    FETCH_SIZE / WRITE_SIZE calibration), then the Llama prefill, scatter and
    decode kernels n times each, eagerly, one dispatch per call."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=DEV)
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    case = W.llama_prefill()
    c = case.cache
    pool = device_pool(c)
    bt = i32(c.block_table)
    k, v = case.tokens.k.to(DEV), case.tokens.v.to(DEV)
    slots, pos = i32(case.tokens.slot_ids), i32(case.tokens.positions)
    q, lens, sid = case.q.to(DEV), i32(case.seq_lens), i32(case.slot_ids)
    for _ in range(n):
        pa.kv_scatter(k, v, slots, pos, pool, bt, c.layer)
    for _ in range(n):
        pa.attn_prefill(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, True, slot_ids=sid)
    del pool
    d = W.llama_decode()
    c = d.cache
    pool = device_pool(c)
    tables = [i32(t) for t in decode_replicas(d, 8)]
    for bt in tables:
        for tok in (d.context, d.new_tokens):
            pa.kv_scatter(tok.k.to(DEV), tok.v.to(DEV), i32(tok.slot_ids), i32(tok.positions), pool,
                          bt, c.layer)
    q, lens, sid = d.q.to(DEV), i32(d.ctx_lens), i32(d.slot_ids)
    ws = pa.decode_workspace(d.B, d.Hq, c.n_kv_heads, d.d, d.max_ctx, DEV)
    for i in range(n):
        pa.attn_decode(q, pool, tables[i % 8], c.layer, lens, c.n_kv_heads, d.scale, d.max_ctx,
                       slot_ids=sid, workspace=ws)
    del pool
    # the long decode (4 x 16384): the whole-page kernel and its merge kernel
    d = W.long_decode()
    c = d.cache
    pool = device_pool(c)
    tables = [i32(t) for t in decode_replicas(d, 4)]
    for bt in tables:
        for tok in (d.context, d.new_tokens):
            pa.kv_scatter(tok.k.to(DEV), tok.v.to(DEV), i32(tok.slot_ids), i32(tok.positions), pool,
                          bt, c.layer)
    q, lens, sid = d.q.to(DEV), i32(d.ctx_lens), i32(d.slot_ids)
    ws = pa.decode_workspace(d.B, d.Hq, c.n_kv_heads, d.d, d.max_ctx, DEV)
    for i in range(n):
        pa.attn_decode(q, pool, tables[i % 4], c.layer, lens, c.n_kv_heads, d.scale, d.max_ctx,
                       slot_ids=sid, workspace=ws)
    torch.cuda.synchronize()
    print(f"kernels-only: {n} launches each", flush=True)


SWEEP_PARTS = ("tiny", "dense", "long_prefill", "long_decode", "decode_d128", "prefill_d128", "chunk", "append",
               "backward", "decode_batch", "cpu")


def sweep(parts=SWEEP_PARTS) -> None:
    """The other configurations' measurements (one line each, then a
    markdown table): the 17-token prompt (latency), the dense FA2-shape grid
    (MHA, d 64 / 128, T 512..16k, B*T = 16k, causal and full), the long dense
    prefill (B=1, T=16384, 16x128, causal), the long decode (4 x 16384), a
    prefix continuation and a mixed prefill + decode batch, the decode append
    of the 64-sequence batch, a release of 8 of its slots, and the backward
    on the FA2 shapes.
    Kernel times are HIP-event averages over graph replays (kernel_time)."""
    rows = []

    def emit(name, us, metric, unit, extra=""):
        rows.append((name, us, metric, unit, extra))
        print(f"sweep: {name}: {us:.2f} us, {metric:.2f} {unit} {extra}", flush=True)

    if "tiny" in parts:
        # 17-token prefill: scatter and prefill separately
        case = W.tiny_prefill()
        c = case.cache
        pool = device_pool(c)
        bt = i32(c.block_table)
        k, v = case.tokens.k.to(DEV), case.tokens.v.to(DEV)
        slots, pos = i32(case.tokens.slot_ids), i32(case.tokens.positions)
        q, lens, sid = case.q.to(DEV), i32(case.seq_lens), i32(case.slot_ids)
        t_sc = kernel_time(lambda: pa.kv_scatter(k, v, slots, pos, pool, bt, c.layer))
        t_pf = kernel_time(lambda: pa.attn_prefill(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale,
                                                   True, slot_ids=sid))
        emit("17-token kv_scatter", t_sc * 1e6, t_sc * 1e6, "us")
        emit("17-token prefill (32/8/64, paged)", t_pf * 1e6, prefill_flops(1, 17, 32, 64, True) / t_pf / 1e9,
             "GFLOP/s")
        del pool

    if "dense" in parts:
        # dense FA2 shapes
        for d, H in W.FA2_HEADS:
            for T in W.FA2_SEQLENS:
                res = {}
                for causal in (False, True):
                    dc = W.fa2_dense(T, d, causal)
                    qd, kd, vd = dc.q.to(DEV), dc.k.to(DEV), dc.v.to(DEV)
                    Od = torch.empty_like(qd)
                    Ld = torch.empty(dc.q.shape[0], H, T, dtype=torch.float32, device=DEV)
                    t = kernel_time(lambda: pa.attn_prefill_dense(qd, kd, vd, dc.scale, causal, out=Od, lse=Ld),
                                    reps=10, trials=3)
                    B = 16384 // T
                    res[causal] = t
                    emit(f"dense d={d} H={H} T={T} B={B} {'causal' if causal else 'full'}", t * 1e6,
                         prefill_flops(B, T, H, d, causal) / t / 1e12, "TFLOP/s")
                    del qd, kd, vd, Od, Ld
                rows[-1] = rows[-1][:4] + (f"full/causal time ratio {res[False] / res[True]:.2f}",)

    if "long_prefill" in parts:
        # long dense prefill
        lc = W.long_prefill()
        ql, kl, vl = lc.q.to(DEV), lc.k.to(DEV), lc.v.to(DEV)
        t = kernel_time(lambda: pa.attn_prefill_dense(ql, kl, vl, lc.scale, True), reps=5, trials=3)
        emit("long prefill B=1 T=16384 16x128 causal (dense)", t * 1e6,
             prefill_flops(1, 16384, 16, 128, True) / t / 1e12, "TFLOP/s")
        del ql, kl, vl

    if "long_decode" in parts:
        # long decode, 4 page-disjoint replicas cycled (537 MB, past the 256 MB MALL)
        dcase = W.long_decode()
        c = dcase.cache
        pool = device_pool(c)
        tables = [i32(tb) for tb in decode_replicas(dcase, 4)]
        for tb in tables:
            for tok in (dcase.context, dcase.new_tokens):
                pa.kv_scatter(tok.k.to(DEV), tok.v.to(DEV), i32(tok.slot_ids), i32(tok.positions), pool, tb,
                              c.layer)
        qd, lens, sid = dcase.q.to(DEV), i32(dcase.ctx_lens), i32(dcase.slot_ids)
        ws = pa.decode_workspace(dcase.B, dcase.Hq, c.n_kv_heads, dcase.d, dcase.max_ctx, DEV)
        t = kernel_time(lambda: [pa.attn_decode(qd, pool, tb, c.layer, lens, c.n_kv_heads, dcase.scale,
                                                dcase.max_ctx, slot_ids=sid, workspace=ws) for tb in tables],
                        reps=4) / len(tables)
        kvb = int(dcase.ctx_lens.sum()) * c.n_kv_heads * dcase.d * 2 * 2
        emit("long decode 4 x 16384 (32/8/64, paged)", t * 1e6, kvb / t / 1e9, "GB/s",
             decode_path_note(dcase.B, dcase.Hq, c.n_kv_heads, dcase.d, dcase.max_ctx))

    if "decode_d128" in parts:
        # the decode batch with head_dim 128: 64 sequences, ctx ~ U[1, 2048], 32/8 heads,
        # 4 page-disjoint replicas cycled (1.1 GB of K/V, past the MALL)
        dcase = W.make_decode("decode_d128", B=64, Hq=32, Hkv=8, d=128, n_pages=20000, seed=0)
        c = dcase.cache
        pool = device_pool(c)
        tables = [i32(tb) for tb in decode_replicas(dcase, 4)]
        for tb in tables:
            for tok in (dcase.context, dcase.new_tokens):
                pa.kv_scatter(tok.k.to(DEV), tok.v.to(DEV), i32(tok.slot_ids), i32(tok.positions), pool, tb,
                              c.layer)
        qd, lens, sid = dcase.q.to(DEV), i32(dcase.ctx_lens), i32(dcase.slot_ids)
        ws = pa.decode_workspace(dcase.B, dcase.Hq, c.n_kv_heads, dcase.d, dcase.max_ctx, DEV)
        t = kernel_time(lambda: [pa.attn_decode(qd, pool, tb, c.layer, lens, c.n_kv_heads, dcase.scale,
                                                dcase.max_ctx, slot_ids=sid, workspace=ws) for tb in tables],
                        reps=4) / len(tables)
        kvb = int(dcase.ctx_lens.sum()) * c.n_kv_heads * dcase.d * 2 * 2
        emit("decode B=64, ctx ~ U[1, 2048] (32/8/128, paged)", t * 1e6, kvb / t / 1e9, "GB/s",
             f"{int(dcase.ctx_lens.sum())} context tokens")
        del pool

    if "prefill_d128" in parts:
        # the Llama prefill shape with head_dim 128 (2 x 2048 tokens, 32/8/128, paged,
        # causal), as two launches and as one (attn_prefill_append)
        pc = W.make_prefill("prefill_d128", B=2, T=2048, Hq=32, Hkv=8, d=128, n_pages=4096, seed=0,
                            scale=1.0 / np.sqrt(128.0))
        c = pc.cache
        pool = device_pool(c)
        bt = i32(c.block_table)
        kk, vv = pc.tokens.k.to(DEV), pc.tokens.v.to(DEV)
        pa.kv_scatter(kk, vv, i32(pc.tokens.slot_ids), i32(pc.tokens.positions), pool, bt, c.layer)
        qq, lens, sid = pc.q.to(DEV), i32(pc.seq_lens), i32(pc.slot_ids)
        fl = prefill_flops(pc.B, pc.T, pc.Hq, pc.d, True)
        t = kernel_time(lambda: pa.attn_prefill(qq, pool, bt, c.layer, lens, c.n_kv_heads, pc.scale, True,
                                                slot_ids=sid))
        emit("prefill 2 x 2048, 32/8/128, paged, causal", t * 1e6, fl / t / 1e12, "TFLOP/s", "attn_prefill")
        kd, vd = kk.view(pc.B, pc.T, c.n_kv_heads, pc.d), vv.view(pc.B, pc.T, c.n_kv_heads, pc.d)
        t = kernel_time(lambda: pa.attn_prefill_append(qq, kd, vd, pool, bt, c.layer, lens, pc.scale, True,
                                                       slot_ids=sid))
        emit("prefill step in one launch, 2 x 2048, 32/8/128 (attn_prefill_append)", t * 1e6, fl / t / 1e12,
             "TFLOP/s", "K/V rows written to the pages in the same launch")
        del pool

    if "decode_batch" in parts:
        # other decode batches of the same mix: 16 to 512 sequences, ctx ~ U[1, 2048],
        # 32/8/64, an 8 GiB pool, 4 page-disjoint replicas cycled
        for Bd in (16, 32, 48, 80, 96, 128, 256, 512):
            dcase = W.make_decode(f"decode_b{Bd}", B=Bd, Hq=32, Hkv=8, d=64, n_pages=4 * W.POOL_PAGES,
                                  seed=Bd, scale=1.0 / 8.0, mbps=128)
            c = dcase.cache
            pool = device_pool(c)
            # enough page-disjoint replicas that the cycled K/V (>= 600 MB) is not
            # served from the 256 MB MALL
            kvb1 = int(dcase.ctx_lens.sum()) * c.n_kv_heads * dcase.d * 2 * 2
            n_rep = max(4, -(-600_000_000 // kvb1))
            tables = [i32(tb) for tb in decode_replicas(dcase, n_rep)]
            for tb in tables:
                for tok in (dcase.context, dcase.new_tokens):
                    pa.kv_scatter(tok.k.to(DEV), tok.v.to(DEV), i32(tok.slot_ids), i32(tok.positions), pool,
                                  tb, c.layer)
            qd, lens, sid = dcase.q.to(DEV), i32(dcase.ctx_lens), i32(dcase.slot_ids)
            ws = pa.decode_workspace(dcase.B, dcase.Hq, c.n_kv_heads, dcase.d, dcase.max_ctx, DEV)
            t = kernel_time(lambda: [pa.attn_decode(qd, pool, tb, c.layer, lens, c.n_kv_heads, dcase.scale,
                                                    dcase.max_ctx, slot_ids=sid, workspace=ws)
                                     for tb in tables], reps=4) / len(tables)
            kvb = int(dcase.ctx_lens.sum()) * c.n_kv_heads * dcase.d * 2 * 2
            emit(f"decode B={Bd}, ctx ~ U[1, 2048] (32/8/64, paged)", t * 1e6, kvb / t / 1e9, "GB/s",
                 f"{int(dcase.ctx_lens.sum())} context tokens, {100 * kvb / t / 1e9 / PEAK_HBM_GBS:.1f}% of HBM; "
                 + decode_path_note(Bd, 32, 8, 64, dcase.max_ctx))
            del pool, tables

    if "chunk" in parts:
        # prefix continuation and a mixed prefill + decode batch (attn_prefill_chunk);
        # FLOPs count every visible (query, key) pair: 4 * d * Hq per pair
        long_chunk = W.make_chunk("chunk_after_16k", B=1, Hq=32, Hkv=8, d=64, n_pages=4096,
                                  kv_lens=[16384 + 128], q_lens=[128], seed=7, scale=1.0 / 8.0, mbps=1040)
        for cc, label in ((W.llama_chunk(), "chunk: 2 x (2048 cached + 2048 new), 32/8/64, causal"),
                          (W.mixed_batch(), "mixed: 2 chunks of 512 + 62 decode rows, 32/8/64"),
                          (long_chunk, "chunk: 128 new after 16384 cached, 32/8/64, causal")):
            c = cc.cache
            pool = device_pool(c)
            bt = i32(c.block_table)
            pa.kv_scatter(cc.tokens.k.to(DEV), cc.tokens.v.to(DEV), i32(cc.tokens.slot_ids),
                          i32(cc.tokens.positions), pool, bt, c.layer)
            qc, kvl, ql, sid = cc.q.to(DEV), i32(cc.seq_lens), i32(cc.q_lens), i32(cc.slot_ids)
            Oc = torch.empty_like(qc)
            Lc = torch.empty(cc.B, cc.Hq, cc.T, dtype=torch.float32, device=DEV)
            t = kernel_time(lambda: pa.attn_prefill(qc, pool, bt, c.layer, kvl, c.n_kv_heads, cc.scale, True,
                                                    slot_ids=sid, out=Oc, lse=Lc, q_lens=ql), reps=10, trials=3)
            pairs = sum(int(q) * (int(k) - int(q)) + int(q) * (int(q) + 1) // 2
                        for q, k in zip(cc.q_lens, cc.seq_lens))
            emit(label, t * 1e6, 4.0 * cc.d * cc.Hq * pairs / t / 1e12, "TFLOP/s",
                 f"{pairs} visible (query, key) pairs per head")
            # the same batch with packed rows (attn_prefill_packed): the host plan is
            # made once (outside the timed region, as one plan serves every layer)
            plan = pa.prefill_packed_plan(cc.q_lens, cc.seq_lens, cc.Hq, c.n_kv_heads, cc.d, True)
            prow = [(b, r) for b in range(cc.B) for r in range(int(cc.q_lens[b]))]
            qp = cc.q[torch.tensor([r[0] for r in prow]), torch.tensor([r[1] for r in prow])].contiguous().to(DEV)
            q_start = i32(np.concatenate([[0], np.cumsum(cc.q_lens)]))
            wsp = plan.workspace()
            Op = torch.empty_like(qp)
            Lp = torch.empty(qp.shape[0], cc.Hq, dtype=torch.float32, device=DEV)
            t = kernel_time(lambda: pa.attn_prefill_packed(qp, pool, bt, c.layer, kvl, q_start, plan, c.n_kv_heads,
                                                           cc.scale, True, slot_ids=sid, workspace=wsp, out=Op,
                                                           lse=Lp), reps=10, trials=3)
            emit(label.replace(":", " (packed rows):", 1), t * 1e6, 4.0 * cc.d * cc.Hq * pairs / t / 1e12,
                 "TFLOP/s", f"{plan.n_work} work items, {plan.n_merge} split row blocks merged")
            del pool, qc, Oc, Lc, qp, Op, Lp, wsp

    if "append" in parts:
        # decode append for the 64-sequence batch: RoPE of K and q, page pops, K/V write
        ac = W.llama_append()
        dc = ac.decode
        c = dc.cache
        pool = device_pool(c)
        bt = i32(ac.block_table)
        free_np = np.full(c.n_pages, -1, np.int32)
        free_np[:ac.top] = ac.free_pages
        free = i32(free_np)
        alloc = pa.new_alloc_state(ac.top, DEV)
        cos_t = torch.from_numpy(ac.cos_t).to(DEV)
        sin_t = torch.from_numpy(ac.sin_t).to(DEV)
        nt = dc.new_tokens
        nk, nv, npos, nsl = nt.k.to(DEV), nt.v.to(DEV), i32(nt.positions), i32(dc.slot_ids)
        qa = dc.q.to(DEV)
        q_out = torch.empty_like(qa)
        t = kernel_time(lambda: pa.kv_append(nk, nv, npos, cos_t, sin_t, pool, bt, c.layer, free, alloc,
                                             slot_ids=nsl, q=qa, q_out=q_out))
        n_open = int(((nt.positions % 16) == 0).sum())
        ab = (2 * nk.numel() + 2 * qa.numel()) * 2 * 2 + dc.B * ac.cos_t.shape[1] * 4 * 2 + n_open * 4
        emit("kv_append B=64 (32/8/64): RoPE of K and q, page pops, K/V write", t * 1e6, ab / t / 1e9, "GB/s",
             f"{n_open} of {dc.B} tokens open a page; {ab} bytes moved")

        # release of 8 of the 64 sequences (one workgroup, in order): graphs of
        # (restore the table and the stack top, release) minus graphs of the restore alone
        bt0, alloc0 = bt.clone(), alloc.clone()
        rel = i32(np.arange(8))
        n_rel = int((ac.block_table[:8] >= 0).sum())

        def restore():
            bt.copy_(bt0)
            alloc.copy_(alloc0)

        def restore_release():
            restore()
            pa.kv_release(rel, bt, free, alloc)

        t_rr = kernel_time(restore_release)
        t_r = kernel_time(restore)
        us = (t_rr - t_r) * 1e6
        emit("kv_release of 8 slots (1 layer x 128 blocks each)", us, n_rel / us, "pages/us",
             f"{n_rel} pages pushed; graph of restore+release minus graph of restore")
        del pool

    if "backward" in parts:
        # backward on the FA2 shapes: FLOPs = 2.5 x forward (the explainer's convention:
        # 5 matrix products against 2); fwd+bwd = 3.5 x forward
        for d, H in W.FA2_HEADS:
            for T in W.FA2_SEQLENS:
                for causal in (False, True):
                    gc = W.fa2_dense(T, d, causal, grad=True)
                    qd, kd, vd, dod = (x.to(DEV) for x in (gc.q, gc.k, gc.v, gc.dout))
                    Od, Ld = pa.attn_prefill_dense(qd, kd, vd, gc.scale, causal)
                    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
                    B = 16384 // T
                    ws = torch.empty(max(int(pa.load().attn_backward_workspace_size(B, T, H)), 16),
                                     dtype=torch.uint8, device=DEV)
                    tb = kernel_time(lambda: pa.attn_backward_dense(qd, kd, vd, Od, dod, Ld, gc.scale, causal,
                                                                    dq=dq, dk=dk, dv=dv, workspace=ws),
                                     reps=5, trials=3)
                    tf = kernel_time(lambda: pa.attn_prefill_dense(qd, kd, vd, gc.scale, causal, out=Od, lse=Ld),
                                     reps=5, trials=3)
                    fwd = prefill_flops(B, T, H, d, causal)
                    emit(f"backward d={d} H={H} T={T} B={B} {'causal' if causal else 'full'}", tb * 1e6,
                         2.5 * fwd / tb / 1e12, "TFLOP/s",
                         f"fwd+bwd {3.5 * fwd / (tf + tb) / 1e12:.1f} TFLOP/s")
                    del qd, kd, vd, dod, Od, Ld, dq, dk, dv, ws

    if "cpu" in parts:
        # the fp64 CPU oracle on the 17-token prompt (whole, every thread and one
        # thread), the dense FA2 grid and the long prefill (64 rows spread
        # evenly over the first sequence's positions, every thread; rate = the
        # sample's FLOPs / its time, whole-case time extrapolated from it) and the
        # long decode (whole, every thread)
        import oracle
        nt = oracle.num_threads()
        host = host_info()
        print(f"sweep: oracle host: {host}", flush=True)
        case = W.tiny_prefill()
        pool = oracle.pool_for(case)
        oracle.scatter_tokens(pool, case.cache, case.tokens)
        fl = prefill_flops(1, 17, 32, 64, True)
        dt, reps = _repeat(lambda: oracle.prefill_case(case, pool=pool), 1.0)
        dt1, reps1 = _one_thread(lambda: _repeat(lambda: oracle.prefill_case(case, pool=pool), 1.0))
        emit(f"oracle, {nt} threads: 17-token prefill (whole)", dt * 1e6, fl / dt / 1e9, "GFLOP/s",
             f"{reps} repeats")
        emit("oracle, 1 thread: 17-token prefill (whole)", dt1 * 1e6, fl / dt1 / 1e9, "GFLOP/s",
             f"{reps1} repeats")
        for d, H in W.FA2_HEADS:
            for T in W.FA2_SEQLENS:
                for causal in (False, True):
                    dc = W.fa2_dense(T, d, causal)
                    B = 16384 // T
                    rws = spread_rows(B, T, 64, seqs=[0])
                    rf = row_flops(rws, T, H, d, causal)
                    dt, reps = _repeat(lambda: oracle.dense_case(dc, rws), 0.3)
                    full = prefill_flops(B, T, H, d, causal)
                    emit(f"oracle, {nt} threads: dense d={d} H={H} T={T} B={B} {'causal' if causal else 'full'}",
                         dt * full / rf * 1e6, rf / dt / 1e9, "GFLOP/s",
                         f"64 rows of sequence 0, {rf / full * 100:.3f}% of the FLOPs; "
                         f"whole case {dt * full / rf:.1f} s extrapolated")
        lc = W.long_prefill()
        rws = spread_rows(1, 16384, 64)
        rf = row_flops(rws, 16384, 16, 128, True)
        full = prefill_flops(1, 16384, 16, 128, True)
        dt, reps = _repeat(lambda: oracle.dense_case(lc, rws), 1.0)
        emit(f"oracle, {nt} threads: long prefill B=1 T=16384 16x128 causal", dt * full / rf * 1e6,
             rf / dt / 1e9, "GFLOP/s",
             f"64 rows spread over the positions, {rf / full * 100:.3f}% of the FLOPs; "
             f"whole case {dt * full / rf:.1f} s extrapolated")
        dcase = W.long_decode()
        dpool = oracle.pool_for(dcase)
        oracle.scatter_tokens(dpool, dcase.cache, dcase.context)
        oracle.scatter_tokens(dpool, dcase.cache, dcase.new_tokens)
        dt, reps = _repeat(lambda: oracle.decode_case(dcase, pool=dpool), 1.0)
        kvb = int(dcase.ctx_lens.sum()) * dcase.cache.n_kv_heads * dcase.d * 2 * 2
        emit(f"oracle, {nt} threads: long decode 4 x 16384 (whole)", dt * 1e6, kvb / dt / 1e9, "GB/s",
             f"{reps} repeats")
        del pool, dpool

    print("\n| workload | time (us) | throughput | note |\n|---|---:|---:|---|")
    for name, us, metric, unit, extra in rows:
        print(f"| {name} | {us:.2f} | {metric:.2f} {unit} | {extra} |")


def main() -> int:
    global SUSTAIN_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sustain", type=float, default=SUSTAIN_S, metavar="S",
                    help="seconds of back-to-back steps after the timed ones, reported as `sustained` (0: off)")
    ap.add_argument("--kernels-only", type=int, default=0, metavar="N",
                    help="launch each dominant kernel N times for a counter run; no JSON")
    ap.add_argument("--sweep", nargs="*", default=None, metavar="PART",
                    help="measure the other configurations instead of the JSON line; parts: "
                         + ", ".join(SWEEP_PARTS) + " (default: all)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    pa.load()
    if args.kernels_only:
        kernels_only(args.kernels_only)
        return 0
    if args.sweep is not None:
        bad = [x for x in args.sweep if x not in SWEEP_PARTS]
        if bad:
            print(f"unknown sweep part(s): {bad}", file=sys.stderr)
            return 2
        sweep(tuple(args.sweep) or SWEEP_PARTS)
        return 0

    SUSTAIN_S = max(0.0, args.sustain)
    p = bench_prefill(args.steps, args.warmup)
    d = bench_decode(args.steps, args.warmup)

    prefill_digest = source_digest("device.h", "prefill.hip")
    decode_digest = source_digest("device.h", "decode.hip")
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
                     "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_of("prefill", prefill_digest),
                     "clock_GHz": round(p["clock_ghz"], 3),
                     "peak_at_clock": round(PEAK_BF16_TFLOPS * p["clock_ghz"] / RATED_CLOCK_GHZ, 1),
                     "frac_at_clock": round(kern_tflops / (PEAK_BF16_TFLOPS * p["clock_ghz"] / RATED_CLOCK_GHZ), 4),
                     "avg_us": round(p["t_kernel"] * 1e6, 3), "alg_bytes": p["alg_bytes"],
                     "single_launch": p["spread"], "source_digest": prefill_digest},
        "context": {"note": "figures the FlashAttention-2 explainer reports on A100 (section Results); "
                            "other hardware, quoted for context, not targets",
                    "fa2_forward_frac_of_peak_a100": [0.50, 0.73],
                    "fa2_training_tflops_per_a100": 225},
        "scatter_us": round(p["t_scatter"] * 1e6, 3),
        "append_step": {"step": "attn_prefill_append (the 4096 prompt tokens written and attended in one launch)",
                        "ms_per_step": round(p["wall_append"] / args.steps * 1e3, 5),
                        "value": round(p["flops"] / (p["wall_append"] / args.steps) / 1e12, 3)},
        "sustained": p["sustained"],
        "decode": {
            "metric": "decode KV-read GB/s", "unit": "GB/s",
            "value": round(d["kv_bytes"] / (d["wall"] / args.steps) / 1e9, 2),
            "ms_per_step": round(d_ms, 5),
            "sustained": d["sustained"],
            "pct_of_hbm_peak": round(100 * d["kv_bytes"] / (d["wall"] / args.steps) / 1e9 / PEAK_HBM_GBS, 2),
            "config": {"workload": "paged decode step, 64 sequences, ctx ~ U[1, 2048]",
                       "batch": dcase.B, "ctx_tokens": d["n_ctx"], "kv_bytes": d["kv_bytes"],
                       "replicas": d["replicas"], "step": "kv_scatter(64 tokens) + attn_decode"},
            "append_step": {"step": "attn_decode_append (the 64 new tokens written and attended in one launch)",
                            "ms_per_step": round(d["wall_append"] / args.steps * 1e3, 5),
                            "value": round(d["kv_bytes"] / (d["wall_append"] / args.steps) / 1e9, 2)},
            "roofline": {"kernel": "decode_kernel<64,4,false>", "bound": "hbm",
                         "achieved": round(d_kern, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(d_kern / PEAK_HBM_GBS, 4),
                         "traffic": traffic_of("decode", decode_digest),
                         "avg_us": round(d["t_kernel"] * 1e6, 3), "alg_bytes": d_alg,
                         "page_granular_bytes": d["page_bytes"],
                         "page_granular_GBs": round(d["page_bytes"] / d["t_kernel"] / 1e9, 2),
                         "single_launch": d["spread"], "source_digest": decode_digest},
        },
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_prefill_baseline(case)
        out["decode"]["cpu_baseline"] = cpu_decode_baseline(dcase)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
