"""attn_prefill (paged) and attn_prefill_dense on the GPU against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (DEV, assert_attn_close, device_pool, i32, prefill_rows_layout, run_prefill,
                      sample_rows, scatter)

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _full_parity(case, what=None):
    O, L, pool = run_prefill(case)
    Oref, Lref, _ = oracle.prefill_case(case)
    B, T, Hq, d = case.q.shape
    # oracle rows are (b, t) in order: [B*T, Hq, d] and [B*T, Hq]
    assert_attn_close(O.reshape(B * T, Hq, d), L.permute(0, 2, 1).reshape(B * T, Hq), Oref, Lref,
                      what=what or case.name)
    return O, L, pool


def test_prefill_tiny_prompt():
    _full_parity(W.tiny_prefill())


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged(Hq, Hkv, d, causal):
    # lengths crossing the 32-row, 64-key and 128-row tile edges, plus empty and 1
    lens = [200, 1, 64, 65, 0, 129]
    case = W.make_prefill("ragged", B=len(lens), T=200, Hq=Hq, Hkv=Hkv, d=d, n_pages=120,
                          seed=Hq + d, seq_lens=lens, causal=causal, n_layers=2, layer=1,
                          n_slots=8, slot_ids=[7, 0, 3, 5, 1, 2], fill_other_layers=True)
    O, L, _ = _full_parity(case)
    assert torch.all(O[4] == 0) and torch.all(torch.isneginf(L[4]))


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (8, 8, 128), (16, 8, 64)])
def test_prefill_writes_every_output(Hq, Hkv, d):
    # O and LSE start as NaN: every element, padding rows (past a sequence's
    # length) and rows of the last partial query tile included, is written
    lens = [77, 3, 0, 100]
    case = W.make_prefill("poisoned", B=len(lens), T=100, Hq=Hq, Hkv=Hkv, d=d, n_pages=40,
                          seed=7 * Hq + d, seq_lens=lens, causal=True)
    c = case.cache
    bt = i32(c.block_table)
    pool = device_pool(c)
    scatter(pool, c, case.tokens, bt)
    q = case.q.to(DEV)
    O = torch.full_like(q, float("nan"))
    L = torch.full((case.B, case.Hq, case.T), float("nan"), dtype=torch.float32, device=DEV)
    pa.attn_prefill(q, pool, bt, c.layer, i32(case.seq_lens), c.n_kv_heads, case.scale, True,
                    slot_ids=i32(case.slot_ids), out=O, lse=L)
    torch.cuda.synchronize()
    assert not torch.isnan(O).any() and not torch.isnan(L).any()
    Oref, Lref, _ = oracle.prefill_case(case)
    B, T = case.B, case.T
    assert_attn_close(O.reshape(B * T, Hq, d), L.permute(0, 2, 1).reshape(B * T, Hq), Oref, Lref,
                      what=case.name)
    for b, n in enumerate(lens):   # padding rows: O = 0, LSE = -inf
        assert torch.all(O[b, n:] == 0) and torch.all(torch.isneginf(L[b, :, n:]))


def _ramped(k: torch.Tensor, pos: torch.Tensor, top: float) -> torch.Tensor:
    """|k| scaled by 1 + top*pos/max(pos): with |q| the scores climb along the keys."""
    ramp = 1.0 + top * pos.float() / max(1, int(pos.max()))
    return (k.float().abs() * ramp.view(-1, *([1] * (k.dim() - 1)))).to(torch.bfloat16)


@pytest.mark.parametrize("top", [15.0, 40.0])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_climbing_scores(top, d, causal):
    """Scores that rise by tens (top=15) to hundreds (top=40) of log2 units from
    one key tile to the next, so the kernel's reference max has to move after
    a row's first tile, sometimes by more than its 2^64 allowance in one step.
    Attention then sits on a few keys, so O is close to single V rows; V is
    scaled by 1/4 to keep |O| in the range the absolute O tolerance is set
    for (P in bf16 bounds the O error by 2^-9 max|V| plus rounding of O)."""
    lens = [300, 257]
    case = W.make_prefill("climbing", B=2, T=300, Hq=8, Hkv=2, d=d, n_pages=64, seed=int(top) + d,
                          seq_lens=lens, causal=causal)
    case.q = case.q.float().abs().to(torch.bfloat16)
    t = case.tokens
    t.k = _ramped(t.k, torch.as_tensor(t.positions), top)
    t.v = (t.v.float() * 0.25).to(torch.bfloat16)
    _full_parity(case)


@pytest.mark.parametrize("d", [64, 128])
def test_dense_climbing_scores(d):
    case = W.make_dense("climbing", B=2, T=330, Hq=8, Hkv=2, d=d, causal=True, seed=5)
    case.q = case.q.float().abs().to(torch.bfloat16)
    pos = torch.arange(case.k.shape[1]).repeat(case.k.shape[0])
    k = _ramped(case.k.reshape(-1, *case.k.shape[2:]), pos, 30.0)
    case.k = k.reshape(case.k.shape)
    case.v = (case.v.float() * 0.25).to(torch.bfloat16)
    _dense_parity(case)


def test_prefill_llama_sampled_rows():
    case = W.llama_prefill()
    O, L, _ = run_prefill(case)
    rows = sample_rows(case.B, case.T, per_seq=48)
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
    Og, Lg = prefill_rows_layout(O, L, rows)
    assert_attn_close(Og, Lg, Oref, Lref, what="llama prefill")


def test_prefill_llama_all_rows():
    """Every row of the full-size prefill (2 x 2048 rows x 32 heads) element by element."""
    case = W.llama_prefill()
    _full_parity(case)


# Rows around the page-offset windows of the paged kernel (a window holds the
# pages of 64 key tiles = 4096 keys): the first and last rows of each window,
# the tile and page edges next to them, and the last rows of the prompt.
_WINDOW_ROWS = [0, 1, 63, 64, 1000, 4094, 4095, 4096, 4097, 4111, 4112, 4159, 4160, 6000, 8190,
                8191, 8192, 8193, 8255, 8256, 8500]


def _long_rows(case, extra=()):
    rows = []
    for b in range(case.B):
        n = int(case.seq_lens[b]) if case.q_lens is None else int(case.q_lens[b])
        ts = {t for t in _WINDOW_ROWS + list(extra) if t < n} | {n - 2, n - 1}
        ts |= set(np.random.default_rng(b).integers(0, n, 12).tolist())
        rows += [(b, t) for t in sorted(t for t in ts if t >= 0)]
    return np.array(rows, np.int32)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_past_one_page_window(causal):
    """Prompts of 9000 and 8500 tokens (141 and 133 key tiles: windows 0-2 of the
    kernel's page offsets), 1024 blocks per sequence in the table, against the
    oracle on rows whose keys reach into each window."""
    case = W.make_prefill("long_paged", B=2, T=9000, Hq=32, Hkv=8, d=64, n_pages=2048, seed=31,
                          seq_lens=[9000, 8500], causal=causal, mbps=1024)
    O, L, _ = run_prefill(case)
    rows = _long_rows(case)
    Oref, Lref, _ = oracle.prefill_case(case, rows=rows)
    Og, Lg = prefill_rows_layout(O, L, rows)
    assert_attn_close(Og, Lg, Oref, Lref, what=case.name)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_missing_page_in_second_window(causal):
    """A missing page among the keys of window 1 (keys 4096-8191) and one in
    window 2: its keys are left out and flagged; rows before, across and after
    it match the oracle, which leaves out the same keys."""
    case = W.make_prefill("hole", B=1, T=9000, Hq=32, Hkv=8, d=64, n_pages=1024, seed=32,
                          causal=causal, mbps=1024)
    _, _, pool = run_prefill(case)
    bt = case.cache.block_table.copy()
    bt[0, 0, 300] = -1        # keys 4800..4815, tile 75
    bt[0, 0, 530] = -1        # keys 8480..8495, tile 132
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O, L = pa.attn_prefill(case.q.to(DEV), pool, i32(bt), 0, i32(case.seq_lens), 8, case.scale,
                           causal, err=err)
    rows = _long_rows(case, extra=(4799, 4800, 4815, 4816, 4830, 8479, 8480, 8496, 8990))
    pool_h = oracle.pool_for(case)
    oracle.scatter_tokens(pool_h, case.cache, case.tokens)
    Oref, Lref, bad = oracle.attn_prefill(case.q, pool_h, case.cache.n_pages, bt, 0, None,
                                          case.seq_lens, 8, case.scale, causal, rows=rows)
    assert bad > 0
    torch.cuda.synchronize()
    assert int(err.item()) == pa.PA_DEVERR_BAD_PAGE
    Og, Lg = prefill_rows_layout(O, L, rows)
    assert_attn_close(Og, Lg, Oref, Lref, what="missing pages in windows 1 and 2")


def test_prefill_deterministic_and_permutation_bitwise():
    a = W.make_prefill("pa", B=2, T=300, Hq=32, Hkv=8, d=64, n_pages=128, seed=21)
    b = W.make_prefill("pb", B=2, T=300, Hq=32, Hkv=8, d=64, n_pages=128, seed=21)
    perm = np.random.default_rng(99).permutation(128).astype(np.int32)
    b.cache.block_table = np.where(a.cache.block_table >= 0, perm[np.maximum(a.cache.block_table, 0)], -1)
    Oa, La, pool = run_prefill(a)
    Oa2, La2, _ = run_prefill(a, pool=pool)
    Ob, Lb, _ = run_prefill(b)
    assert torch.equal(Oa, Oa2) and torch.equal(La, La2)
    assert torch.equal(Oa, Ob) and torch.equal(La, Lb)


def test_prefill_zero_query_running_mean():
    case = W.make_prefill("zq", B=1, T=130, Hq=32, Hkv=8, d=64, n_pages=16, seed=4)
    case.q = torch.zeros_like(case.q)
    O, L, _ = run_prefill(case)
    expect = torch.log(torch.arange(1, 131, dtype=torch.float32))
    assert (L[0].cpu() - expect[None, :]).abs().max() <= 1e-3
    _full_parity(case)


def test_prefill_worked_example_row():
    d = 64
    case = W.make_prefill("fa2", B=1, T=4, Hq=1, Hkv=1, d=d, n_pages=4, seed=2, scale=1 / 8)
    q = torch.zeros(1, 4, 1, d)
    q[..., 0] = 8.0
    k = torch.zeros(4, 1, d)
    k[:, 0, 0] = torch.tensor([1.0, 2.0, 3.0, 0.0])
    v = torch.zeros(4, 1, d)
    v[:, 0, 0] = torch.tensor([10.0, 20.0, 30.0, 0.0])
    case.q = q.to(torch.bfloat16)
    case.tokens.k, case.tokens.v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    O, L, _ = run_prefill(case)
    assert abs(float(O[0, 3, 0, 0]) - 24.9265) <= 0.125
    assert abs(float(L[0, 0, 3]) - 3.440190) <= 1e-3
    assert abs(float(L[0, 0, 1]) - (2 + math.log(1 + math.exp(-1)))) <= 1e-3


def test_prefill_missing_page_is_flagged_and_skipped():
    case = W.make_prefill("bad", B=1, T=100, Hq=32, Hkv=8, d=64, n_pages=16, seed=8)
    _, _, pool = run_prefill(case)
    bt = case.cache.block_table.copy()
    bt[0, 0, 3] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    O, L = pa.attn_prefill(case.q.to(DEV), pool, i32(bt), 0, i32(case.seq_lens), 8, case.scale,
                           err=err)
    pool_h = oracle.pool_for(case)
    oracle.scatter_tokens(pool_h, case.cache, case.tokens)
    Oref, Lref, bad = oracle.attn_prefill(case.q, pool_h, 16, bt, 0, None, case.seq_lens, 8,
                                          case.scale, True)
    assert bad > 0
    torch.cuda.synchronize()
    assert int(err.item()) & pa.PA_DEVERR_BAD_PAGE
    # every row still sees keys 0..47, so every row is compared
    assert_attn_close(O[0], L[0].T, Oref, Lref, what="missing page")


# ------------------------------------------------------------------- dense

def _dense_parity(case, rows=None):
    O, L = pa.attn_prefill_dense(case.q.to(DEV), case.k.to(DEV), case.v.to(DEV), case.scale,
                                 case.causal)
    Oref, Lref = oracle.dense_case(case, rows=rows)
    B, T, Hq, d = case.q.shape
    if rows is None:
        assert_attn_close(O.reshape(B * T, Hq, d), L.permute(0, 2, 1).reshape(B * T, Hq), Oref,
                          Lref, what=case.name)
    else:
        Og, Lg = prefill_rows_layout(O, L, rows)
        assert_attn_close(Og, Lg, Oref, Lref, what=case.name)
    return O, L


@pytest.mark.parametrize("d,H,Hkv", [(64, 8, 8), (128, 4, 4), (64, 16, 4), (128, 8, 2), (64, 32, 2), (128, 16, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_small(d, H, Hkv, causal):
    _dense_parity(W.make_dense("dense", B=2, T=333, Hq=H, Hkv=Hkv, d=d, causal=causal, seed=d + H))


@pytest.mark.parametrize("T", W.FA2_SEQLENS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_fa2_shapes_sampled(T, d, causal):
    case = W.fa2_dense(T, d, causal)
    rows = sample_rows(case.q.shape[0], T, per_seq=max(4, 64 // case.q.shape[0]))
    if len(rows) > 160:
        rows = rows[np.random.default_rng(0).permutation(len(rows))[:160]]
    _dense_parity(case, rows=rows)


def test_dense_long_prefill_sampled():
    case = W.long_prefill()
    rows = sample_rows(1, case.q.shape[1], per_seq=40)
    _dense_parity(case, rows=rows)


def test_paged_equals_dense_bitwise():
    """Same keys, same tiles: the paged and the dense instance give identical bits."""
    p = W.make_prefill("p", B=2, T=200, Hq=32, Hkv=8, d=64, n_pages=64, seed=13)
    Op, Lp, _ = run_prefill(p)
    k = p.tokens.k.reshape(2, 200, 8, 64).to(DEV)
    v = p.tokens.v.reshape(2, 200, 8, 64).to(DEV)
    Od, Ld = pa.attn_prefill_dense(p.q.to(DEV), k, v, p.scale, True)
    assert torch.equal(Op, Od) and torch.equal(Lp, Ld)
