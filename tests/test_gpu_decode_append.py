"""attn_decode_append on the GPU: one launch writes every sequence's new token to
its page and attends to the whole context.  The pool after the call equals the
pool after kv_scatter of the new tokens byte for byte, and O, LSE match the
oracle (which scatters the new tokens and decodes) element by element."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def new_rows(case):
    """k_new, v_new [B, Hkv, d]: the new token of every sequence (zeros where the
    context is empty and nothing is written)."""
    c = case.cache
    k = torch.zeros(case.B, c.n_kv_heads, c.head_dim, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    has = np.flatnonzero(np.asarray(case.ctx_lens) > 0)
    k[torch.as_tensor(has, dtype=torch.long)] = case.new_tokens.k
    v[torch.as_tensor(has, dtype=torch.long)] = case.new_tokens.v
    return k.to(DEV), v.to(DEV)


def run_both(case, bt_host=None):
    """(O, LSE, pool) of attn_decode_append, and the pool after kv_scatter of the
    new tokens (both pools start from the cached context)."""
    c = case.cache
    bt = i32(c.block_table if bt_host is None else bt_host)
    pool = device_pool(c)
    scatter(pool, c, case.context, i32(c.block_table))
    ref_pool = pool.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref_err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scatter(ref_pool, c, case.new_tokens, bt, err=ref_err)
    k_new, v_new = new_rows(case)
    mc = max(int(np.max(case.ctx_lens)), 1)
    O, L = pa.attn_decode_append(case.q.to(DEV), k_new, v_new, pool, bt, c.layer, i32(case.ctx_lens),
                                 c.n_kv_heads, case.scale, mc, slot_ids=i32(case.slot_ids), err=err)
    torch.cuda.synchronize()
    return O, L, pool, ref_pool, int(err.item()), int(ref_err.item())


CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700, 1000, 0]


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (8, 8, 64), (16, 1, 64), (32, 16, 64), (64, 8, 64),
                                      (32, 8, 128), (16, 1, 128), (16, 4, 128), (64, 8, 128)])
def test_append_ragged_contexts(Hq, Hkv, d):
    case = W.make_decode("append_ragged", B=len(CTX), Hq=Hq, Hkv=Hkv, d=d, n_pages=200, ctx_lens=CTX,
                         seed=Hq + d + 1, n_layers=2, layer=1, n_slots=len(CTX) + 3,
                         slot_ids=np.random.default_rng(3).permutation(len(CTX) + 3)[:len(CTX)])
    O, L, pool, ref_pool, e, re_ = run_both(case)
    assert e == 0 and re_ == 0
    assert torch.equal(pool, ref_pool), "pool differs from kv_scatter's"
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(O, L, Oref, Lref, what=case.name)
    assert torch.all(O[-1] == 0) and torch.all(torch.isneginf(L[-1]))


@pytest.mark.parametrize("d", [64, 128])
def test_append_long_contexts_split(d):
    """Contexts split across workgroups: only the split holding the new token adds it."""
    case = W.make_decode("append_long", B=4, Hq=32, Hkv=8, d=d, n_pages=2048, ctx_lens=[16384, 9000, 70, 1],
                         max_ctx=16384, seed=31 + d, mbps=1024)
    assert pa.decode_splits(4, 32, 8, d, 16384) > 1
    O, L, pool, ref_pool, e, _ = run_both(case)
    assert e == 0
    assert torch.equal(pool, ref_pool)
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(O, L, Oref, Lref, what=case.name)


def test_append_llama_batch_equals_scatter_then_decode():
    """The 64-sequence batch: the fused step against kv_scatter + attn_decode (the
    same bytes in the pool, O and LSE within the tolerance) and the oracle."""
    case = W.llama_decode(seed=7)
    O, L, pool, ref_pool, e, _ = run_both(case)
    assert e == 0 and torch.equal(pool, ref_pool)
    c = case.cache
    O2, L2 = pa.attn_decode(case.q.to(DEV), ref_pool, i32(c.block_table), c.layer, i32(case.ctx_lens),
                            c.n_kv_heads, case.scale, 2048, slot_ids=i32(case.slot_ids))
    assert (O.float() - O2.float()).abs().max().item() <= 2e-2
    assert (L - L2).abs().max().item() <= 1e-3
    Oref, Lref, _ = oracle.decode_case(case)
    assert_attn_close(O, L, Oref, Lref, what=case.name)


def test_append_missing_page_of_the_new_token():
    """The new token's page is missing: flagged, nothing written, the token left
    out of the attention (as kv_scatter + attn_decode would)."""
    case = W.make_decode("append_hole", B=2, Hq=32, Hkv=8, d=64, n_pages=64, ctx_lens=[40, 90], seed=8)
    bt = case.cache.block_table.copy()
    bt[case.slot_ids[1], 0, (90 - 1) // 16] = -1     # the page of sequence 1's new token
    O, L, pool, ref_pool, e, re_ = run_both(case, bt_host=bt)
    assert e & pa.PA_DEVERR_BAD_PAGE and re_ & pa.PA_DEVERR_BAD_PAGE
    assert torch.equal(pool, ref_pool)
    pool_h = oracle.pool_for(case)
    oracle.scatter_tokens(pool_h, case.cache, case.context)
    holed = dataclasses.replace(case.cache, block_table=bt)
    assert oracle.scatter_tokens(pool_h, holed, case.new_tokens) == 1   # sequence 1's is not written
    Oref, Lref, bad = oracle.attn_decode(case.q, pool_h, 64, bt, 0, case.slot_ids, case.ctx_lens, 8,
                                         case.scale)
    assert bad > 0
    assert_attn_close(O, L, Oref, Lref, what="new token on a missing page")
