"""The hot path captured in a HIP graph, as a serving loop replays it: before each
replay new queries are written into the captured input buffer, eager work and a
synchronisation run between replays, and every replay gives the same bits as an
eager call on the same inputs (the kernels allocate nothing, clear nothing with
memsets, and keep no state across calls).  One replay is also checked against
the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, prefill_rows_layout, sample_rows, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _new_q(shape, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=gen).to(torch.bfloat16).to(DEV)


def _replays(q_buf, graph, outs, eager):
    """Replay with a fresh q each time; compare with an eager call bit for bit."""
    for r in range(REPLAYS):
        q_buf.copy_(_new_q(tuple(q_buf.shape), 1000 + r))
        graph.replay()
        torch.cuda.synchronize()
        _ = (outs[0].float() * 2).sum().item()          # eager work between replays
        ref = eager(q_buf.clone())
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r}: graph result differs from the eager call"


def test_prefill_graph_replays():
    case = W.make_prefill("graph_prefill", B=2, T=300, Hq=32, Hkv=8, d=64, n_pages=200, seed=3,
                          scale=0.125)
    c = case.cache
    bt = i32(c.block_table)
    pool = device_pool(c)
    scatter(pool, c, case.tokens, bt)
    lens, slots = i32(case.seq_lens), i32(case.slot_ids)
    q_buf = case.q.to(DEV).clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q_buf)
    lse = torch.empty(2, 32, 300, dtype=torch.float32, device=DEV)

    def call(q, o=None, l=None):
        return pa.attn_prefill(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, True, slot_ids=slots,
                               err=err, out=o, lse=l)

    graph, outs = _capture(lambda: call(q_buf, out, lse))
    _replays(q_buf, graph, outs, call)
    # the last replay against the oracle on sampled rows
    rows = sample_rows(2, 300, 8, seed=1)
    case.q = q_buf.cpu()
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
    Og, Lg = prefill_rows_layout(out, lse, rows)
    assert_attn_close(Og, Lg, Oref, Lref, what="prefill, last graph replay")
    assert int(err.item()) == 0


def test_decode_with_splits_graph_replays():
    """Long contexts: the split partials and the combine kernel inside the graph."""
    case = W.make_decode("graph_decode", B=3, Hq=32, Hkv=8, d=64, n_pages=4096, ctx_lens=[16384, 9000, 70],
                         max_ctx=16384, seed=4, scale=0.125, mbps=1024)
    c = case.cache
    bt = i32(c.block_table)
    pool = device_pool(c)
    scatter(pool, c, case.context, bt)
    scatter(pool, c, case.new_tokens, bt)
    assert pa.decode_workspace_size(3, 32, 8, 64, 16384) > 0
    ws = pa.decode_workspace(3, 32, 8, 64, 16384, DEV)
    lens, slots = i32(case.ctx_lens), i32(case.slot_ids)
    q_buf = case.q.to(DEV).clone()
    out = torch.empty_like(q_buf)
    lse = torch.empty(3, 32, dtype=torch.float32, device=DEV)

    def call(q, o=None, l=None):
        return pa.attn_decode(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, 16384, slot_ids=slots,
                              workspace=ws, out=o, lse=l)

    graph, outs = _capture(lambda: call(q_buf, out, lse))
    _replays(q_buf, graph, outs, call)
    case.q = q_buf.cpu()
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(out, lse, Oref, Lref, what="decode, last graph replay")


def test_packed_with_merges_graph_replays():
    """The mixed batch on packed rows: split pieces, partial tiles in the workspace
    and the merge kernel inside the graph."""
    case = W.mixed_batch(seed=5)
    c = case.cache
    bt = i32(c.block_table)
    pool = device_pool(c)
    scatter(pool, c, case.tokens, bt)
    ql = np.asarray(case.q_lens, np.int64)
    rows = np.array([(b, t) for b in range(case.B) for t in range(int(ql[b]))], np.int32)
    q_start = i32(np.concatenate([[0], np.cumsum(ql)]))
    plan = pa.prefill_packed_plan(case.q_lens, case.seq_lens, case.Hq, c.n_kv_heads, case.d, case.causal)
    assert plan.n_merge > 0
    ws = plan.workspace()
    lens, slots = i32(case.seq_lens), i32(case.slot_ids)
    q_buf = case.q[torch.as_tensor(rows[:, 0], dtype=torch.long),
                   torch.as_tensor(rows[:, 1], dtype=torch.long)].contiguous().to(DEV)
    out = torch.empty_like(q_buf)
    lse = torch.empty(q_buf.shape[0], case.Hq, dtype=torch.float32, device=DEV)

    def call(q, o=None, l=None):
        return pa.attn_prefill_packed(q, pool, bt, c.layer, lens, q_start, plan, c.n_kv_heads, case.scale,
                                      case.causal, slot_ids=slots, workspace=ws, out=o, lse=l)

    graph, outs = _capture(lambda: call(q_buf, out, lse))
    _replays(q_buf, graph, outs, call)
    qp = q_buf.cpu()
    qpad = torch.zeros_like(case.q)
    qpad[torch.as_tensor(rows[:, 0], dtype=torch.long), torch.as_tensor(rows[:, 1], dtype=torch.long)] = qp
    case.q = qpad
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
    assert_attn_close(out, lse, Oref, Lref, what="packed, last graph replay")


def test_decode_append_graph_replays():
    """The one-launch decode step in a graph: before each replay new queries and
    new K/V rows are written into the captured buffers; every replay writes the
    same pool bytes and gives the same O, LSE as an eager call, and the last one
    matches kv_scatter's pool and the oracle (split contexts and the combine
    kernel included)."""
    import dataclasses
    case = W.make_decode("graph_append", B=3, Hq=32, Hkv=8, d=64, n_pages=4096, ctx_lens=[16384, 9000, 70],
                         max_ctx=16384, seed=6, scale=0.125, mbps=1024)
    c = case.cache
    bt = i32(c.block_table)
    pool = device_pool(c)
    scatter(pool, c, case.context, bt)
    ws = pa.decode_workspace(3, 32, 8, 64, 16384, DEV)
    lens, slots = i32(case.ctx_lens), i32(case.slot_ids)
    q_buf = case.q.to(DEV).clone()
    k_buf = case.new_tokens.k.to(DEV).clone()
    v_buf = case.new_tokens.v.to(DEV).clone()
    out = torch.empty_like(q_buf)
    lse = torch.empty(3, 32, dtype=torch.float32, device=DEV)

    def call(q, k, v, o=None, l=None):
        return pa.attn_decode_append(q, k, v, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, 16384,
                                     slot_ids=slots, workspace=ws, out=o, lse=l)

    graph, outs = _capture(lambda: call(q_buf, k_buf, v_buf, out, lse))
    for r in range(REPLAYS):
        q_buf.copy_(_new_q(tuple(q_buf.shape), 2000 + r))
        k_buf.copy_(_new_q(tuple(k_buf.shape), 3000 + r))
        v_buf.copy_(_new_q(tuple(v_buf.shape), 4000 + r))
        graph.replay()
        torch.cuda.synchronize()
        pool_after = pool.clone()
        _ = (out.float() * 2).sum().item()              # eager work between replays
        ref = call(q_buf.clone(), k_buf.clone(), v_buf.clone())
        torch.cuda.synchronize()
        assert torch.equal(pool, pool_after), f"replay {r}: the eager call wrote other pool bytes"
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r}: graph result differs from the eager call"
    # the last replay: the pool as kv_scatter of the last new rows leaves it, O and LSE as the oracle's
    new = dataclasses.replace(case.new_tokens, k=k_buf.cpu(), v=v_buf.cpu())
    ref_pool = device_pool(c)
    scatter(ref_pool, c, case.context, bt)
    scatter(ref_pool, c, new, bt)
    torch.cuda.synchronize()
    assert torch.equal(pool, ref_pool)
    case.q = q_buf.cpu()
    case.new_tokens = new
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(out, lse, Oref, Lref, what="decode append, last graph replay")
