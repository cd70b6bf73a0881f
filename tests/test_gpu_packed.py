"""attn_prefill_packed on the GPU against the oracle: packed query rows (prompt
chunks after cached prefixes, whole prompts, decode rows) run by a host plan
whose long row blocks are split across workgroups and merged, every row
element by element."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, run_prefill, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def packed_rows(case):
    """(b, t) of every query row in packed order, and q_start [B + 1]."""
    ql = np.asarray(case.q_lens, np.int64)
    rows = np.array([(b, t) for b in range(case.B) for t in range(int(ql[b]))], np.int32).reshape(-1, 2)
    return rows, np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)


def run_packed(case, pool=None, bt=None, err=None, plan=None):
    c = case.cache
    rows, q_start = packed_rows(case)
    if bt is None:
        bt = i32(c.block_table)
    if pool is None:
        pool = device_pool(c)
        scatter(pool, c, case.tokens, bt)
    if plan is None:
        plan = pa.prefill_packed_plan(case.q_lens, case.seq_lens, case.Hq, c.n_kv_heads, case.d, case.causal)
    q = case.q[torch.as_tensor(rows[:, 0], dtype=torch.long), torch.as_tensor(rows[:, 1], dtype=torch.long)]
    O, L = pa.attn_prefill_packed(q.contiguous().to(DEV), pool, bt, c.layer, i32(case.seq_lens), i32(q_start),
                                  plan, c.n_kv_heads, case.scale, case.causal, slot_ids=i32(case.slot_ids),
                                  err=err)
    return O, L, pool, rows, plan


def _parity(case, what=None):
    O, L, pool, rows, plan = run_packed(case)
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
    assert_attn_close(O, L, Oref, Lref, what=what or case.name)
    return O, L, pool, rows, plan


KV = [300, 129, 64, 65, 17, 1, 250, 96, 40, 200]
QL = [37, 64, 1, 65, 16, 1, 250, 0, 33, 129]


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (8, 8, 64), (16, 8, 64), (8, 1, 64),
                                      (32, 8, 128), (16, 16, 128), (8, 1, 128), (32, 2, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_packed_ragged(Hq, Hkv, d, causal):
    n = len(KV)
    case = W.make_chunk("packed_ragged", B=n, Hq=Hq, Hkv=Hkv, d=d, n_pages=160, kv_lens=KV, q_lens=QL,
                        seed=Hq + d, causal=causal, n_layers=2, layer=1, n_slots=n + 2,
                        slot_ids=np.random.default_rng(2).permutation(n + 2)[:n], mbps=20)
    _parity(case)


def test_packed_mixed_batch_every_row():
    """Two 512-token chunks (after 1000 and 3000 cached tokens) and 62 decode rows:
    every packed row."""
    _parity(W.mixed_batch())


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (16, 8, 128), (8, 1, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_packed_split_pieces_past_one_window(Hq, Hkv, d, causal):
    """300-row chunks after 9000 / 13000 cached tokens and a decode row after 6000:
    pieces start in every window of 64 key tiles (the page offsets are reloaded
    from the piece's first tile); every row against the oracle."""
    case = W.make_chunk("packed_long", B=3, Hq=Hq, Hkv=Hkv, d=d, n_pages=2048, kv_lens=[9300, 13300, 6001],
                        q_lens=[300, 300, 1], seed=43 + d, causal=causal, mbps=1024)
    _, _, _, _, plan = _parity(case)
    items = plan.host[:6 * plan.n_work].reshape(-1, 6)
    assert plan.n_merge > 0 and (items[:, 3] >= 64).any() and (items[:, 3] % 64 != 0).any()


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (16, 8, 128), (8, 1, 64), (8, 8, 64), (32, 2, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_packed_narrow_row_blocks_split(Hq, Hkv, d, causal):
    """Decode rows and short row-block tails (at most 32/HW rows: one wave holds
    every head of the block) after long contexts, cut into many pieces (little
    other work, so the share per CU is small) and merged: every row."""
    case = W.make_chunk("packed_narrow", B=4, Hq=Hq, Hkv=Hkv, d=d, n_pages=2048,
                        kv_lens=[16000, 9005, 50, 4500], q_lens=[1, 5, 1, 37], seed=71 + d, causal=causal,
                        mbps=1024)
    _, _, _, _, plan = _parity(case)
    assert plan.n_merge > 0


def test_packed_missing_pages_in_later_windows():
    """A missing page in window 1 and one in window 2 under split pieces: their keys
    are left out and flagged, like the oracle does."""
    case = W.make_chunk("packed_hole", B=2, Hq=32, Hkv=8, d=64, n_pages=2048, kv_lens=[9000, 600],
                        q_lens=[400, 1], seed=51, causal=True, mbps=1024)
    c = case.cache
    pool = device_pool(c)
    scatter(pool, c, case.tokens)
    bt = c.block_table.copy()
    bt[0, 0, 300] = -1
    bt[0, 0, 530] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O, L, _, rows, plan = run_packed(case, pool=pool, bt=i32(bt), err=err)
    assert plan.n_merge > 0
    pool_h = oracle.pool_for(case)
    oracle.scatter_tokens(pool_h, c, case.tokens)
    Oref, Lref, bad = oracle.attn_prefill(case.q, pool_h, c.n_pages, bt, c.layer, case.slot_ids, case.seq_lens,
                                          c.n_kv_heads, case.scale, True, rows=rows, q_lens=case.q_lens)
    assert bad > 0
    torch.cuda.synchronize()
    assert int(err.item()) == pa.PA_DEVERR_BAD_PAGE
    assert_attn_close(O, L, Oref, Lref, what="packed, missing pages in windows 1 and 2")


def test_packed_unsplit_equals_chunk_bitwise():
    """A batch the plan does not split: every packed row equals attn_prefill_chunk's
    padded row bit for bit (the same kernel code for an unsplit row block)."""
    n = len(KV)
    case = W.make_chunk("packed_vs_chunk", B=n, Hq=32, Hkv=8, d=64, n_pages=160, kv_lens=KV, q_lens=QL,
                        seed=5, causal=True, mbps=20)
    O, L, pool, rows, plan = run_packed(case)
    assert plan.n_merge == 0
    Oc, Lc, _ = run_prefill(case, pool=pool)
    b = torch.as_tensor(rows[:, 0], dtype=torch.long, device=DEV)
    t = torch.as_tensor(rows[:, 1], dtype=torch.long, device=DEV)
    assert torch.equal(O, Oc[b, t]) and torch.equal(L, Lc[b, :, t])


def test_packed_plan_reused_and_deterministic():
    """One plan, two runs (as every layer of a step would): identical bits."""
    case = W.mixed_batch(seed=2)
    O1, L1, pool, rows, plan = run_packed(case)
    O2, L2, _, _, _ = run_packed(case, pool=pool, plan=plan)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_packed_bad_plan_item_is_flagged_and_skipped():
    """A work item whose partial slot lies past the workspace (forced from the host):
    flagged with PA_DEVERR_BAD_PLAN, nothing written out of bounds, the other
    sequences' rows unaffected."""
    case = W.make_chunk("packed_bad", B=2, Hq=32, Hkv=8, d=64, n_pages=2048, kv_lens=[9000, 300],
                        q_lens=[64, 300], seed=61, causal=True, mbps=1024)
    plan = pa.prefill_packed_plan(case.q_lens, case.seq_lens, 32, 8, 64, True)
    host = plan.host.copy()
    items = host[:6 * plan.n_work].reshape(-1, 6)
    bad = int(np.flatnonzero((items[:, 0] == 0) & (items[:, 5] >= 0))[0])
    items[bad, 5] = 1 << 30
    bad_plan = pa.PackedPlan(host, plan.n_work, plan.n_merge, plan.workspace_bytes, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O, L, _, rows, _ = run_packed(case, err=err, plan=bad_plan)
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_PLAN
    keep = rows[:, 0] == 1
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows[keep])
    k = torch.as_tensor(np.flatnonzero(keep), dtype=torch.long, device=DEV)
    assert_attn_close(O[k], L[k], Oref, Lref, what="rows of the sequence with a good plan")
