"""attn_prefill_chunk on the GPU against the oracle: prompt chunks continuing a
cached prefix (queries = the last q_len of kv_len cached tokens) and mixed
prefill + decode batches, element by element."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (DEV, assert_attn_close, i32, prefill_rows_layout, run_prefill, sample_rows)

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _parity(case, rows=None, what=None):
    O, L, pool = run_prefill(case)
    if rows is None:
        Oref, Lref, _ = oracle.prefill_case(case)
        Og, Lg = O.reshape(-1, case.Hq, case.d), L.permute(0, 2, 1).reshape(-1, case.Hq)
    else:
        Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
        Og, Lg = prefill_rows_layout(O, L, rows)
    assert_attn_close(Og, Lg, Oref, Lref, what=what or case.name)
    return O, L, pool


# chunk lengths around page (16), tile (64) and query-tile (32 / 128) edges, prefixes of
# every phase, single rows (decode), whole prompts and empty chunks
KV = [300, 129, 64, 65, 17, 1, 250, 96, 40, 200]
QL = [37, 64, 1, 65, 16, 1, 250, 0, 33, 129]


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (8, 8, 64), (16, 8, 64), (8, 1, 64),
                                      (32, 8, 128), (16, 16, 128), (8, 1, 128), (32, 2, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_ragged(Hq, Hkv, d, causal):
    n = len(KV)
    case = W.make_chunk("ragged", B=n, Hq=Hq, Hkv=Hkv, d=d, n_pages=160, kv_lens=KV, q_lens=QL,
                        seed=Hq + d, causal=causal, n_layers=2, layer=1, n_slots=n + 2,
                        slot_ids=np.random.default_rng(2).permutation(n + 2)[:n], mbps=20)
    _parity(case)


def test_chunk_llama_prefix_continuation():
    """2 sequences, 2048 cached tokens each, a 2048-token chunk: sampled rows incl. tile edges."""
    case = W.llama_chunk()
    _parity(case, rows=sample_rows(case.B, case.T, 40, seed=3))


def test_mixed_prefill_and_decode_batch():
    """Two 512-token chunks and 62 decode rows in one call; decode rows also equal attn_decode."""
    case = W.mixed_batch()
    rows = np.concatenate([sample_rows(2, case.T, 40, seed=4),
                           np.stack([np.arange(2, 64), np.zeros(62, np.int64)], 1)]).astype(np.int32)
    O, L, pool = _parity(case, rows=rows)
    # the decode rows through attn_decode on the same pool: same values within tolerance
    c = case.cache
    qd = case.q[2:, 0].to(DEV).contiguous()
    Od, Ld = pa.attn_decode(qd, pool, i32(c.block_table), c.layer, i32(case.seq_lens[2:]), c.n_kv_heads,
                            case.scale, int(case.seq_lens[2:].max()), slot_ids=i32(case.slot_ids[2:]))
    dO = (Od.float() - O[2:, 0].float()).abs().max().item()
    dL = (Ld - L[2:, :, 0]).abs().max().item()
    assert dO <= 2e-2 and dL <= 1e-3, (dO, dL)


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_after_long_prefix(causal):
    """300-token chunks after 9000 and 13000 cached tokens (keys in windows 0-3 of
    the kernel's page offsets, 4096 keys each), 1024 blocks per sequence in the
    table: every chunk row against the oracle."""
    case = W.make_chunk("chunk_long", B=2, Hq=32, Hkv=8, d=64, n_pages=2048, kv_lens=[9300, 13300],
                        q_lens=[300, 300], seed=41, causal=causal, mbps=1024)
    _parity(case)


def test_chunk_whole_prompt_equals_attn_prefill():
    """q_len = kv_len for every sequence: attn_prefill_chunk gives attn_prefill's output bit for bit."""
    case = W.make_chunk("whole", B=3, Hq=32, Hkv=8, d=64, n_pages=80, kv_lens=[200, 77, 128],
                        q_lens=[200, 77, 128], seed=6)
    O1, L1, pool = run_prefill(case)
    c = case.cache
    O2, L2 = pa.attn_prefill(case.q.to(DEV), pool, i32(c.block_table), c.layer, i32(case.seq_lens),
                             c.n_kv_heads, case.scale, True, slot_ids=i32(case.slot_ids))
    assert torch.equal(O1, O2) and torch.equal(L1.nan_to_num(), L2.nan_to_num())


def test_chunk_flags_bad_query_length():
    """q_len > kv_len is clamped and flagged; the other sequences are unaffected."""
    case = W.make_chunk("bad", B=2, Hq=8, Hkv=2, d=64, n_pages=20, kv_lens=[40, 20], q_lens=[10, 20],
                        seed=7)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O, L, pool = run_prefill(case)
    c = case.cache
    pa.attn_prefill(case.q.to(DEV), pool, i32(c.block_table), c.layer, i32([40, 15]), c.n_kv_heads,
                    case.scale, True, slot_ids=i32(case.slot_ids), err=err, q_lens=i32([10, 20]))
    torch.cuda.synchronize()
    assert int(err.item()) == pa.PA_DEVERR_BAD_POS
