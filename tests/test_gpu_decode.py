"""attn_decode on the GPU against the oracle (element by element)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, run_decode, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _parity(case, what=None):
    O, L, _ = run_decode(case)
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(O, L, Oref, Lref, what=what or case.name)
    return O, L


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (8, 8, 64), (16, 8, 64), (64, 8, 64),
                                      (16, 1, 64), (32, 8, 128), (8, 8, 128), (16, 1, 128),
                                      (48, 12, 64), (32, 16, 64), (16, 4, 128)])
def test_decode_ragged_contexts(Hq, Hkv, d):
    # lengths around page (16), chunk (32) and split boundaries, plus an empty context
    ctx = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700, 1000, 0]
    case = W.make_decode("ragged", B=len(ctx), Hq=Hq, Hkv=Hkv, d=d, n_pages=200, ctx_lens=ctx,
                         seed=Hq + d, n_layers=2, layer=1, n_slots=len(ctx) + 3,
                         slot_ids=np.random.default_rng(1).permutation(len(ctx) + 3)[:len(ctx)])
    O, L = _parity(case)
    assert torch.all(O[-1] == 0) and torch.all(torch.isneginf(L[-1]))


@pytest.mark.parametrize("B", [6, 72, 128, 129, 300, 520])
def test_decode_batch_sizes_with_tied_lengths(B):
    # many equal context lengths (ties in the longest-first order), batches
    # whose ranking is shared by 64 and 4 lanes per sequence, the largest
    # ranked batch (128) and batches above it (identity order)
    ctx = np.random.default_rng(B).choice([1, 17, 33, 64], size=B)
    case = W.make_decode("ties", B=B, Hq=32, Hkv=8, d=64, n_pages=4 * B + 8, ctx_lens=ctx,
                         seed=B)
    _parity(case)


def test_decode_llama_batch():
    _parity(W.llama_decode())


def test_decode_long_context():
    _parity(W.long_decode())


def test_decode_d128_long_contexts_split():
    """d=128 (one-page chunks): contexts split across workgroups and merged by the
    combine kernel, next to a short one and a one-token one."""
    case = W.make_decode("long128", B=4, Hq=32, Hkv=8, d=128, n_pages=2048, ctx_lens=[16384, 9000, 70, 1],
                         max_ctx=16384, seed=21, mbps=1024)
    assert pa.decode_splits(4, 32, 8, 128, 16384) > 1
    _parity(case)


def test_decode_d128_llama_shaped_batch():
    """64 sequences, contexts U[1, 2048], 32/8/128: every (sequence, head)."""
    _parity(W.make_decode("b64_d128", B=64, Hq=32, Hkv=8, d=128, n_pages=9000, max_ctx=2048, seed=22,
                          mbps=128))


def test_decode_single_split_and_many_splits_agree():
    """A long context split many ways equals the oracle; so does a short one (no combine)."""
    for ctx in ([3000], [40]):
        _parity(W.make_decode("split", B=1, Hq=32, Hkv=8, d=64, n_pages=256, ctx_lens=ctx, seed=4))


def test_decode_worked_example():
    """The FA2 worked example (scores 1,2,3,0; values 10,20,30,0) as a decode call:
    bf16(24.9265) = 24.875, so O is checked to one bf16 ulp (0.125), LSE to 1e-3."""
    d = 64
    q = torch.zeros(1, 1, d)
    q[0, 0, 0] = 8.0
    k = torch.zeros(4, 1, d)
    k[:, 0, 0] = torch.tensor([1.0, 2.0, 3.0, 0.0])
    v = torch.zeros(4, 1, d)
    v[:, 0, 0] = torch.tensor([10.0, 20.0, 30.0, 0.0])
    case = W.make_decode("fa2", B=1, Hq=1, Hkv=1, d=d, n_pages=8, ctx_lens=[4], seed=3, scale=1 / 8)
    case.q = q.to(torch.bfloat16)
    case.context.k, case.context.v = k[:3].to(torch.bfloat16), v[:3].to(torch.bfloat16)
    case.new_tokens.k, case.new_tokens.v = k[3:].to(torch.bfloat16), v[3:].to(torch.bfloat16)
    O, L, _ = run_decode(case)
    assert abs(float(O[0, 0, 0]) - 24.9265) <= 0.125
    assert abs(float(L[0, 0]) - 3.440190) <= 1e-3
    # the same scores with values scaled by 1/32: normal tolerance applies
    case.context.v = (v[:3] / 32).to(torch.bfloat16)
    case.new_tokens.v = (v[3:] / 32).to(torch.bfloat16)
    _parity(case, "fa2/32")


def test_decode_zero_query_is_mean():
    case = W.make_decode("zq", B=3, Hq=32, Hkv=8, d=64, n_pages=64, ctx_lens=[1, 50, 300], seed=9)
    case.q = torch.zeros_like(case.q)
    O, L, _ = run_decode(case)
    for b, c in enumerate(case.ctx_lens):
        assert torch.allclose(L[b].cpu(), torch.full((32,), math.log(c)), atol=1e-3)
    _parity(case)


def test_decode_page_permutation_bitwise():
    a = W.make_decode("pa", B=8, Hq=32, Hkv=8, d=64, n_pages=512, max_ctx=700, seed=5)
    b = W.make_decode("pb", B=8, Hq=32, Hkv=8, d=64, n_pages=512, max_ctx=700, seed=5)
    perm = np.random.default_rng(77).permutation(512).astype(np.int32)
    b.cache.block_table = np.where(a.cache.block_table >= 0, perm[np.maximum(a.cache.block_table, 0)], -1)
    Oa, La, _ = run_decode(a)
    Ob, Lb, _ = run_decode(b)
    assert torch.equal(Oa, Ob) and torch.equal(La, Lb)


def test_decode_deterministic_and_poison_free():
    case = W.llama_decode(seed=1)
    O1, L1, pool = run_decode(case)
    O2, L2, _ = run_decode(case, pool=pool)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.isfinite(O1.float()).all() and torch.isfinite(L1).all()


def test_decode_equals_last_prefill_row():
    p = W.make_prefill("p", B=1, T=300, Hq=32, Hkv=8, d=64, n_pages=64, seed=12)
    pool = device_pool(p.cache)
    bt = i32(p.cache.block_table)
    scatter(pool, p.cache, p.tokens, bt)
    Op, Lp = pa.attn_prefill(p.q.to(DEV), pool, bt, 0, i32(p.seq_lens), 8, p.scale)
    Od, Ld = pa.attn_decode(p.q[:, -1].contiguous().to(DEV), pool, bt, 0, i32([300]), 8, p.scale, 300)
    assert (Od[0].float() - Op[0, -1].float()).abs().max() <= 2e-2
    assert (Ld[0] - Lp[0, :, -1]).abs().max() <= 1e-3


@pytest.mark.parametrize("d", [64, 128])
def test_decode_missing_page_is_flagged_and_skipped(d):
    case = W.make_decode("bad", B=2, Hq=32, Hkv=8, d=d, n_pages=64, ctx_lens=[90, 40], seed=6)
    Oref0, Lref0, pool_h = oracle.decode_case(case)
    O, L, pool = run_decode(case)
    bt = case.cache.block_table.copy()
    bt[0, 0, 2] = -1                   # tokens 32..47 of sequence 0 lose their page
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O2, L2 = pa.attn_decode(case.q.to(DEV), pool, i32(bt), 0, i32(case.ctx_lens), 8, case.scale,
                            90, slot_ids=i32(case.slot_ids), err=err)
    Oref, Lref, bad = oracle.attn_decode(case.q, pool_h, 64, bt, 0, case.slot_ids, case.ctx_lens,
                                         8, case.scale)
    assert bad == 16 * 32
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_PAGE
    assert_attn_close(O2, L2, Oref, Lref, what="missing page")


def test_decode_bad_length_is_flagged():
    case = W.make_decode("len", B=2, Hq=32, Hkv=8, d=64, n_pages=64, ctx_lens=[20, 30], seed=6)
    _, _, pool = run_decode(case)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.attn_decode(case.q.to(DEV), pool, i32(case.cache.block_table), 0, i32([20, 3000]), 8,
                   case.scale, 30, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_POS


def test_decode_workspace_reused_across_shapes():
    """One workspace, sized for the largest of three shapes and filled with NaN
    bytes before every call (its contents on entry must not matter), serves:
    long contexts split across workgroups (their partials in the workspace), a
    ragged batch, and two short contexts."""
    cases = [W.long_decode(),
             W.make_decode("ragged", B=18, Hq=32, Hkv=8, d=64, n_pages=200,
                           ctx_lens=[1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700, 1000, 0],
                           seed=3),
             W.make_decode("short", B=2, Hq=32, Hkv=8, d=64, n_pages=16, ctx_lens=[40, 7], seed=4)]
    n = max(pa.decode_workspace_size(c.B, c.Hq, c.cache.n_kv_heads, c.d, max(c.max_ctx, 1)) for c in cases)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    for case in cases:
        c = case.cache
        pool = device_pool(c)
        bt = i32(c.block_table)
        scatter(pool, c, case.context, bt)
        scatter(pool, c, case.new_tokens, bt)
        ws.view(torch.int16)[: n // 2].fill_(0x7FC0)   # bf16 / fp32 quiet-NaN bytes
        O, L = pa.attn_decode(case.q.to(DEV), pool, bt, c.layer, i32(case.ctx_lens), c.n_kv_heads,
                              case.scale, max(case.max_ctx, 1), slot_ids=i32(case.slot_ids), workspace=ws)
        Oref, Lref, _ = oracle.decode_case(case)
        assert_attn_close(O, L, Oref, Lref, what=case.name)


def test_decode_whole_pages_missing_pages_at_piece_edges():
    """The whole-page kernel: 5 sequences (1 to 5700 tokens, 805 pages over 256
    workgroups: pieces of 3 or 4 pages, so most sequences are cut into many
    pieces) with missing pages at the first page of a sequence, inside a piece,
    at piece boundaries and on the last, partial page; O and LSE against the
    oracle, the flag raised, the pieces merged."""
    ctx = [3000, 17, 4100, 1, 5700]
    case = W.make_decode("wp_bad", B=5, Hq=32, Hkv=8, d=64, n_pages=1024, ctx_lens=ctx, seed=21, mbps=512)
    assert pa.decode_whole_pages(5, 32, 8, 64, 5700)
    Oref0, Lref0, pool_h = oracle.decode_case(case)
    O, L, pool = run_decode(case)
    assert_attn_close(O, L, Oref0, Lref0, what="whole pages, all present")
    bt = case.cache.block_table.copy()
    for b, blk in ((0, 0), (0, 93), (0, 94), (2, 40), (2, 41), (2, 42), (2, 256), (4, 1), (4, 356)):
        bt[b, 0, blk] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O2, L2 = pa.attn_decode(case.q.to(DEV), pool, i32(bt), 0, i32(case.ctx_lens), 8, case.scale,
                            5700, slot_ids=i32(case.slot_ids), err=err)
    Oref, Lref, bad = oracle.attn_decode(case.q, pool_h, 1024, bt, 0, case.slot_ids, case.ctx_lens,
                                         8, case.scale)
    assert bad > 0
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_PAGE
    assert_attn_close(O2, L2, Oref, Lref, what="whole pages, missing pages")
