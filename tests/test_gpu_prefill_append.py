"""attn_prefill_append on the GPU: one launch writes every prompt token's K/V row
to its page and runs the prefill on the rows of the inputs.  The pool after the
call equals the pool after kv_scatter of the prompt tokens byte for byte; O and
LSE equal attn_prefill's on that pool bit for bit (errors included) and match
the oracle element by element."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def dense_kv(case, pad=float("nan")):
    """k, v [B, T, Hkv, d] of the case's prompt tokens; rows past a sequence's
    length hold NaN (the call must not read them)."""
    B, T = case.B, case.T
    Hkv, d = case.cache.n_kv_heads, case.cache.head_dim
    k = torch.full((B, T, Hkv, d), pad, dtype=torch.bfloat16)
    v = torch.full_like(k, pad)
    bi = np.repeat(np.arange(B), np.asarray(case.seq_lens, np.int64))
    ti = np.asarray(case.tokens.positions, np.int64)
    k[torch.as_tensor(bi), torch.as_tensor(ti)] = case.tokens.k
    v[torch.as_tensor(bi), torch.as_tensor(ti)] = case.tokens.v
    return k, v


def both_paths(case, k, v, seq_lens, slot_ids, bt_host, tokens):
    """(O, LSE, pool, err) of attn_prefill_append and of kv_scatter(tokens) +
    attn_prefill, both from the same starting pool."""
    c = case.cache
    bt = i32(bt_host)
    q = case.q.to(DEV)
    pool_a = device_pool(c)
    err_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    Oa, La = pa.attn_prefill_append(q, k.to(DEV), v.to(DEV), pool_a, bt, c.layer, i32(seq_lens), case.scale,
                                    case.causal, slot_ids=i32(slot_ids), err=err_a)
    pool_b = device_pool(c)
    err_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    scatter(pool_b, c, tokens, bt, err=err_b)
    Ob, Lb = pa.attn_prefill(q, pool_b, bt, c.layer, i32(seq_lens), c.n_kv_heads, case.scale, case.causal,
                             slot_ids=i32(slot_ids), err=err_b)
    torch.cuda.synchronize()
    return (Oa, La, pool_a, int(err_a.item())), (Ob, Lb, pool_b, int(err_b.item()))


def assert_same(a, b, what):
    Oa, La, pa_, ea = a
    Ob, Lb, pb, eb = b
    assert ea == eb, f"{what}: error bits {ea:#x} against {eb:#x}"
    assert torch.equal(pa_, pb), f"{what}: pool differs from kv_scatter's"
    assert torch.equal(Oa, Ob), f"{what}: O differs from attn_prefill's"
    assert torch.equal(La, Lb), f"{what}: LSE differs from attn_prefill's"


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_append_ragged(Hq, Hkv, d, causal):
    lens = [200, 1, 64, 65, 0, 129]
    case = W.make_prefill("append_ragged", B=len(lens), T=200, Hq=Hq, Hkv=Hkv, d=d, n_pages=120,
                          seed=Hq + d + 5, seq_lens=lens, causal=causal, n_layers=2, layer=1,
                          n_slots=8, slot_ids=[7, 0, 3, 5, 1, 2], fill_other_layers=True)
    k, v = dense_kv(case)
    a, b = both_paths(case, k, v, case.seq_lens, case.slot_ids, case.cache.block_table, case.tokens)
    assert a[3] == 0
    assert_same(a, b, case.name)
    Oref, Lref, _ = oracle.prefill_case(case)
    B, T = case.B, case.T
    assert_attn_close(a[0].reshape(B * T, Hq, d), a[1].permute(0, 2, 1).reshape(B * T, Hq), Oref, Lref,
                      what=case.name)


def test_prefill_append_llama_batch():
    """The 2 x 2048-token batch: the pool and O, LSE of the two-launch step, bit for bit."""
    case = W.llama_prefill(seed=11)
    k, v = dense_kv(case)
    a, b = both_paths(case, k, v, case.seq_lens, case.slot_ids, case.cache.block_table, case.tokens)
    assert a[3] == 0
    assert_same(a, b, case.name)


def test_prefill_append_missing_page():
    """A page missing from the table: flagged, its rows not written and its keys
    left out of the attention, as kv_scatter + attn_prefill do."""
    case = W.make_prefill("append_hole", B=2, T=150, Hq=32, Hkv=8, d=64, n_pages=40, seed=21,
                          seq_lens=[150, 90])
    bt = case.cache.block_table.copy()
    bt[case.slot_ids[0], 0, 3] = -1          # keys 48..63 of sequence 0
    bt[case.slot_ids[1], 0, 5] = 10 ** 6     # keys 80..89 of sequence 1: past the pool
    k, v = dense_kv(case)
    a, b = both_paths(case, k, v, case.seq_lens, case.slot_ids, bt, case.tokens)
    assert a[3] & pa.PA_DEVERR_BAD_PAGE
    assert_same(a, b, "missing pages")
    holed = dataclasses.replace(case.cache, block_table=bt)
    pool_h = oracle.pool_for(case)
    assert oracle.scatter_tokens(pool_h, holed, case.tokens) == 16 + 10   # the rows on the two pages
    Oref, Lref, bad = oracle.attn_prefill(case.q, pool_h, holed.n_pages, bt, holed.layer, case.slot_ids,
                                          case.seq_lens, holed.n_kv_heads, case.scale, case.causal)
    assert bad > 0
    assert_attn_close(a[0].reshape(2 * 150, 32, 64), a[1].permute(0, 2, 1).reshape(2 * 150, 32), Oref, Lref,
                      what="missing pages")


def test_prefill_append_bad_slot_and_lengths():
    """A slot outside the table and lengths past the table's reach or past T:
    flagged and clamped as kv_scatter + attn_prefill flag and clamp them."""
    case = W.make_prefill("append_bad", B=4, T=48, Hq=32, Hkv=8, d=64, n_pages=16, seed=31,
                          seq_lens=[32, 20, 10, 5], mbps=2, n_slots=4)
    gen = torch.Generator().manual_seed(5)
    k = torch.randn(4, 48, 8, 64, generator=gen).to(torch.bfloat16)
    v = torch.randn(4, 48, 8, 64, generator=gen).to(torch.bfloat16)
    seq_lens = np.array([40, 20, 10, 60], np.int32)    # 40 > 2 pages; 60 > T
    slot_ids = np.array([0, 9, 2, 3], np.int32)        # slot 9 is outside the table
    # the two-launch step: the tokens the prompts name (positions < min(len, T))
    bi = np.concatenate([np.full(min(int(n), 48), b_) for b_, n in enumerate(seq_lens)])
    ti = np.concatenate([np.arange(min(int(n), 48)) for n in seq_lens])
    tokens = W.TokenBatch(k=k[torch.as_tensor(bi), torch.as_tensor(ti)].contiguous(),
                          v=v[torch.as_tensor(bi), torch.as_tensor(ti)].contiguous(),
                          slot_ids=slot_ids[bi].astype(np.int32), positions=ti.astype(np.int32))
    a, b = both_paths(case, k, v, seq_lens, slot_ids, case.cache.block_table, tokens)
    assert a[3] & pa.PA_DEVERR_BAD_POS and a[3] & pa.PA_DEVERR_BAD_SLOT
    assert_same(a, b, "bad slot and lengths")
    assert torch.all(a[0][1] == 0) and torch.all(torch.isneginf(a[1][1]))


def test_prefill_append_long_prompt_past_one_window():
    """A 9000-token prompt (key tiles past the first 64, whose pages the paged
    instance reads in a second window) with a missing page in that second
    window: the same pool, flags and O, LSE as the two launches, and sampled
    rows whose keys span the windows against the oracle."""
    from gpu_util import sample_rows
    T = 9000
    case = W.make_prefill("append_long", B=1, T=T, Hq=32, Hkv=8, d=64, n_pages=700, seed=41, mbps=600)
    bt = case.cache.block_table.copy()
    bt[case.slot_ids[0], 0, 300] = -1        # keys 4800..4815
    k, v = dense_kv(case)
    a, b = both_paths(case, k, v, case.seq_lens, case.slot_ids, bt, case.tokens)
    assert a[3] & pa.PA_DEVERR_BAD_PAGE
    assert_same(a, b, "long prompt")
    rows = sample_rows(1, T, 24, seed=3)
    rows = np.unique(np.concatenate([rows, np.array([[0, 4799], [0, 4800], [0, 4815], [0, 4816], [0, 8191],
                                                      [0, 8192]], np.int32)]), axis=0)
    holed = dataclasses.replace(case.cache, block_table=bt)
    pool_h = oracle.pool_for(case)
    assert oracle.scatter_tokens(pool_h, holed, case.tokens) == 16
    Oref, Lref, bad = oracle.attn_prefill(case.q, pool_h, holed.n_pages, bt, holed.layer, case.slot_ids,
                                          case.seq_lens, holed.n_kv_heads, case.scale, True, rows)
    assert bad > 0
    Og = a[0][0, torch.as_tensor(rows[:, 1], dtype=torch.long)]
    Lg = a[1][0][:, torch.as_tensor(rows[:, 1], dtype=torch.long)].T
    assert_attn_close(Og, Lg, Oref, Lref, what="long prompt, sampled rows")
