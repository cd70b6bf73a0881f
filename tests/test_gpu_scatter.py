"""kv_scatter on the GPU against the oracle's scatter: whole pool, byte for byte."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, device_pool, i32, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _pool_bytes(pool: torch.Tensor) -> np.ndarray:
    return pool.cpu().numpy()


def _check_case(cache, batches):
    pool = device_pool(cache)
    ref = oracle.new_pool(cache.n_pages, cache.n_kv_heads, cache.head_dim, cache.page_fill)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for tok in batches:
        scatter(pool, cache, tok, err=err)
        assert oracle.scatter_tokens(ref, cache, tok) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = _pool_bytes(pool)
    assert got.shape == ref.shape
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, f"{diff.size} bytes differ, first at byte {diff[:4]}"


def test_scatter_tiny_prompt():
    c = W.tiny_prefill()
    _check_case(c.cache, [c.tokens])


@pytest.mark.parametrize("Hkv,d", [(8, 64), (2, 128), (1, 64)])
def test_scatter_ragged_multi_layer(Hkv, d):
    c = W.make_prefill("sc", B=3, T=70, Hq=Hkv, Hkv=Hkv, d=d, n_pages=80, seed=3,
                       seq_lens=[70, 1, 33], n_layers=3, layer=2, n_slots=5, slot_ids=[4, 0, 2],
                       page_fill=0xBEEF)
    _check_case(c.cache, [c.tokens])


def test_scatter_llama_prompt_full_pool():
    c = W.llama_prefill()
    _check_case(c.cache, [c.tokens])


def test_scatter_decode_append_full_pool():
    c = W.llama_decode()
    _check_case(c.cache, [c.context, c.new_tokens])


def test_scatter_flags_missing_pages_and_leaves_pool():
    c = W.make_prefill("bad", B=1, T=40, Hq=8, Hkv=8, d=64, n_pages=8, seed=2, page_fill=0x1357)
    bt = c.cache.block_table.copy()
    bt[0, 0, 1] = -1           # tokens 16..31 lose their page
    bt_dev = i32(bt)
    pool = device_pool(c.cache)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scatter(pool, c.cache, c.tokens, bt=bt_dev, err=err)
    ref = oracle.new_pool(8, 8, 64, 0x1357)
    skipped = oracle.kv_scatter(ref, 8, c.tokens.k, c.tokens.v, c.tokens.slot_ids,
                                c.tokens.positions, bt, 0, 8, 64)
    assert skipped == 16
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_PAGE
    assert np.array_equal(_pool_bytes(pool), ref)


def test_scatter_flags_bad_slot_and_position():
    c = W.make_prefill("bad", B=1, T=20, Hq=8, Hkv=8, d=64, n_pages=4, seed=2)
    pool = device_pool(c.cache)
    before = _pool_bytes(pool).copy()
    bt = i32(c.cache.block_table)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    k, v = c.tokens.k[:2].to(DEV), c.tokens.v[:2].to(DEV)
    pa.kv_scatter(k, v, i32([7, 0]), i32([0, 5000]), pool, bt, 0, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == pa.PA_DEVERR_BAD_SLOT | pa.PA_DEVERR_BAD_POS
    assert np.array_equal(_pool_bytes(pool), before)
