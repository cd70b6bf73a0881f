"""Pins of the oracle's chunked prefill (queries = the last q_len of kv_len cached
tokens, aligned to the end of the sequence).

The pages only treat q_len == kv_len (tiny-vllm part 3: prefill writes fresh
pages); the reading used is that query row t of a chunk is the token at
position kv_len - q_len + t, with the same causal rule as the whole prompt.
Each pin ties the chunk to something already pinned or to a direct formula:
the same rows of the whole-prompt prefill, the decode call (q_len 1), the
q = 0 closed form, and a numpy evaluation on contiguous K/V.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(causal=True, Hq=8, Hkv=2, d=64, seed=5):
    return W.make_chunk("ch", B=5, Hq=Hq, Hkv=Hkv, d=d, n_pages=60, seed=seed, causal=causal,
                        kv_lens=[40, 37, 17, 64, 9], q_lens=[40, 5, 1, 33, 0], n_layers=2, layer=1,
                        n_slots=7, slot_ids=[6, 0, 3, 2, 5])


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_rows_equal_whole_prompt_rows(oracle_lib, causal):
    """Row t of a chunk equals row kv_len - q_len + t of the whole prompt (same draws)."""
    ch = _case(causal)
    full = W.make_prefill("ch", B=5, T=64, Hq=8, Hkv=2, d=64, n_pages=60, seed=5, causal=causal,
                          seq_lens=[40, 37, 17, 64, 9], n_layers=2, layer=1, n_slots=7,
                          slot_ids=[6, 0, 3, 2, 5])
    assert torch.equal(ch.tokens.k, full.tokens.k)
    Oc, Lc, _ = oracle_lib.prefill_case(ch)
    Of, Lf, _ = oracle_lib.prefill_case(full)
    Oc, Lc = Oc.reshape(5, ch.T, 8, 64), Lc.reshape(5, ch.T, 8)
    Of, Lf = Of.reshape(5, 64, 8, 64), Lf.reshape(5, 64, 8)
    for b in range(5):
        ql, kv = int(ch.q_lens[b]), int(ch.seq_lens[b])
        assert np.array_equal(Oc[b, :ql], Of[b, kv - ql:kv])
        assert np.array_equal(Lc[b, :ql], Lf[b, kv - ql:kv])
        assert np.all(Oc[b, ql:] == 0) and np.all(np.isneginf(Lc[b, ql:]))


def test_chunk_single_row_is_decode(oracle_lib):
    """q_len 1: the query at kv_len - 1 sees every cached key, which is the decode call."""
    ch = W.make_chunk("one", B=3, Hq=8, Hkv=2, d=64, n_pages=40, seed=8, kv_lens=[1, 50, 129],
                      q_lens=[1, 1, 1], mbps=9)
    Oc, Lc, pool = oracle_lib.prefill_case(ch)
    c = ch.cache
    Od, Ld, bad = oracle_lib.attn_decode(ch.q[:, 0], pool, c.n_pages, c.block_table, c.layer,
                                         ch.slot_ids, ch.seq_lens, c.n_kv_heads, ch.scale)
    assert bad == 0
    assert np.array_equal(Oc.reshape(3, 8, 64), Od) and np.array_equal(Lc.reshape(3, 8), Ld)


def test_chunk_zero_query_closed_form(oracle_lib):
    """q = 0: every score is 0, so row t is the mean of V over positions 0..off+t and
    LSE = ln(off + t + 1), off = kv_len - q_len."""
    ch = W.make_chunk("z", B=2, Hq=4, Hkv=4, d=64, n_pages=20, seed=3, kv_lens=[50, 33],
                      q_lens=[20, 7])
    ch.q = torch.zeros_like(ch.q)
    O, L, _ = oracle_lib.prefill_case(ch)
    O, L = O.reshape(2, ch.T, 4, 64), L.reshape(2, ch.T, 4)
    v = ch.tokens.v.float().numpy().astype(np.float64)
    start = 0
    for b in range(2):
        kv, ql = int(ch.seq_lens[b]), int(ch.q_lens[b])
        vb = v[start:start + kv]
        start += kv
        for t in range(ql):
            p = kv - ql + t
            assert np.allclose(O[b, t], vb[:p + 1].mean(0), rtol=0, atol=1e-12)
            assert np.allclose(L[b, t], math.log(p + 1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_matches_numpy_direct(oracle_lib, causal):
    """Direct numpy softmax on contiguous K/V (no block table) for every row of every chunk."""
    ch = _case(causal, Hq=4, Hkv=1, seed=11)
    O, L, _ = oracle_lib.prefill_case(ch)
    O, L = O.reshape(5, ch.T, 4, 64), L.reshape(5, ch.T, 4)
    k = ch.tokens.k.float().numpy().astype(np.float64)
    v = ch.tokens.v.float().numpy().astype(np.float64)
    q = ch.q.float().numpy().astype(np.float64)
    start = 0
    for b in range(5):
        kv, ql = int(ch.seq_lens[b]), int(ch.q_lens[b])
        kb, vb = k[start:start + kv, 0], v[start:start + kv, 0]
        start += kv
        for t in range(ql):
            n = (kv - ql + t + 1) if causal else kv
            for h in range(4):
                s = ch.scale * (kb[:n] @ q[b, t, h])
                m = s.max()
                w = np.exp(s - m)
                assert np.allclose(O[b, t, h], (w @ vb[:n]) / w.sum(), rtol=0, atol=1e-12)
                assert abs(L[b, t, h] - (m + math.log(w.sum()))) < 1e-12
