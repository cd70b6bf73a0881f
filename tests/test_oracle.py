"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself re-typed: each checks a value the
pages print (tests/golden), a closed form, an invariant, a special case, or a
brute-force evaluation that takes a different route (contiguous K/V, no block
table, numpy/scipy primitives).
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads as W
from conftest import read_golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

D = 64


def _bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _pages_table(n_tokens, n_pages, seed, mbps=None):
    """Block table [1][1][mbps] placing one sequence on random pages."""
    rng = np.random.default_rng(seed)
    nb = -(-n_tokens // 16)
    mbps = mbps or max(nb, 1)
    bt = np.full((1, 1, mbps), -1, np.int32)
    bt[0, 0, :nb] = rng.permutation(n_pages)[:nb]
    return bt


def _decode_rows(oracle, q_row, k_rows, v_rows, scale, seed=0, n_pages=16):
    """Run the oracle's paged decode for one sequence with Hq = Hkv = 1."""
    n = k_rows.shape[0]
    bt = _pages_table(n, n_pages, seed)
    pool = oracle.new_pool(n_pages, 1, D, W.BF16_QNAN)
    assert oracle.kv_scatter(pool, n_pages, k_rows.reshape(n, 1, D), v_rows.reshape(n, 1, D),
                             np.zeros(n, np.int32), np.arange(n, dtype=np.int32), bt, 0, 1, D) == 0
    O, L, bad = oracle.attn_decode(q_row.reshape(1, 1, D), pool, n_pages, bt, 0, None,
                                   np.array([n], np.int32), 1, scale)
    assert bad == 0
    return O[0, 0], L[0, 0]


def _score_encoding(scores, values=None, q_mult=1.0, shift=None):
    """q, K, V (bf16) whose scaled scores are exactly bf16(scores) (+ shift)."""
    n = len(scores)
    q = np.zeros(D, np.float32)
    q[0] = q_mult
    k = np.zeros((n, D), np.float32)
    k[:, 0] = scores
    if shift is not None:
        q[1] = shift
        k[:, 1] = 1.0
    if values is None:                      # one-hot rows: O[j] is the weight of key j
        v = np.eye(n, D, dtype=np.float32)
    else:
        v = np.zeros((n, D), np.float32)
        v[:, 0] = values
    return _bf16(q), _bf16(k), _bf16(v)


# ---------------------------------------------------------------- worked example

def test_worked_example_matches_printed_numbers(oracle_lib):
    g = read_golden("fa2_worked_example.txt")
    tol = {k: float(v[-1]) for k, v in g.items()}
    num = {k: [float(x) for x in v[:-1]] for k, v in g.items()}
    s, vals = num["scores"], num["values"]
    # encode with head_dim 64 and scale 1/8: q = 8 e0, k_j = s_j e0 (all exact in bf16)
    q, k, v = _score_encoding(s, values=vals, q_mult=8.0)
    O, L = _decode_rows(oracle_lib, q, k, v, 1.0 / 8.0)
    assert abs(O[0] - num["O"][0]) <= tol["O"]
    assert abs(L - num["L"][0]) <= tol["L"]
    assert np.all(O[1:] == 0)
    # weights: the same scores against one-hot values
    q, k, v = _score_encoding(s, q_mult=8.0)
    Ow, Lw = _decode_rows(oracle_lib, q, k, v, 1.0 / 8.0, seed=3)
    np.testing.assert_allclose(Ow[:4], num["weights"], atol=tol["weights"], rtol=0)
    # the final statistics: L = m + ln l with m = 3, l = 1.553
    assert num["final_max"][0] + math.log(num["final_l"][0]) == pytest.approx(Lw, abs=tol["L"])


def test_worked_example_block_one_is_causal_row_one(oracle_lib):
    """Causal prefill row 1 sees exactly the first block (scores 1, 2): its
    statistics are the page's block-1 intermediates m = 2, l = 1.368 and
    O~ = 23.68, i.e. O = O~ / l and LSE = m + ln l."""
    g = read_golden("fa2_worked_example.txt")
    num = {k: [float(x) for x in v[:-1]] for k, v in g.items()}
    s, vals = num["scores"], num["values"]
    n = len(s)
    # prefill with T = 4, query row t has q_t = 8 e0 for every t; scale 1/8
    q = np.zeros((1, n, 1, D), np.float32)
    q[..., 0] = 8.0
    k = np.zeros((n, 1, D), np.float32)
    k[:, 0, 0] = s
    v = np.zeros((n, 1, D), np.float32)
    v[:, 0, 0] = vals
    bt = _pages_table(n, 8, seed=5)
    pool = oracle_lib.new_pool(8, 1, D, W.BF16_QNAN)
    assert oracle_lib.kv_scatter(pool, 8, _bf16(k), _bf16(v), np.zeros(n, np.int32),
                                 np.arange(n, dtype=np.int32), bt, 0, 1, D) == 0
    O, L, bad = oracle_lib.attn_prefill(_bf16(q), pool, 8, bt, 0, None, np.array([n], np.int32),
                                        1, 1.0 / 8.0, True)
    assert bad == 0
    m1, l1, o1 = num["block1_max"][0], num["block1_l"][0], num["block1_otilde"][0]
    assert O[1, 0, 0] == pytest.approx(o1 / l1, abs=0.01)
    assert L[1, 0] == pytest.approx(m1 + math.log(l1), abs=0.0006)
    # row 3 is the full example
    assert O[3, 0, 0] == pytest.approx(num["O"][0], abs=0.005)
    assert L[3, 0] == pytest.approx(num["L"][0], abs=0.0006)
    # row 0 sees only key 0: O = v0 exactly, LSE = s0
    assert O[0, 0, 0] == vals[0] and L[0, 0] == s[0]


def _blockwise(scores, values, block):
    """FA2 forward recurrence over key blocks (test-side emulation, fp64): keep
    the unnormalised output and l, rescale both when the running max grows,
    divide once at the end; returns (O, L, trace)."""
    m, l, o = -math.inf, 0.0, 0.0
    trace = []
    for i in range(0, len(scores), block):
        sb = np.asarray(scores[i:i + block], float)
        vb = np.asarray(values[i:i + block], float)
        m_new = max(m, float(sb.max()))
        corr = math.exp(m - m_new) if m > -math.inf else 0.0
        o_rescaled = o * corr
        p = np.exp(sb - m_new)
        l = l * corr + float(p.sum())
        o = o_rescaled + float((p * vb).sum())
        m = m_new
        trace.append((m, l, o_rescaled, o))
    return o / l, m + math.log(l), trace


def test_blockwise_recurrence_reproduces_printed_intermediates(oracle_lib):
    g = read_golden("fa2_worked_example.txt")
    num = {k: [float(x) for x in v[:-1]] for k, v in g.items()}
    tol = {k: float(v[-1]) for k, v in g.items()}
    O, L, tr = _blockwise(num["scores"], num["values"], 2)
    assert tr[0][0] == num["block1_max"][0]
    assert tr[0][1] == pytest.approx(num["block1_l"][0], abs=tol["block1_l"])
    assert tr[0][3] == pytest.approx(num["block1_otilde"][0], abs=tol["block1_otilde"])
    assert tr[1][2] == pytest.approx(num["rescaled_otilde"][0], abs=tol["rescaled_otilde"])
    assert tr[1][3] == pytest.approx(num["block2_otilde"][0], abs=tol["block2_otilde"])
    assert tr[1][1] == pytest.approx(num["final_l"][0], abs=tol["final_l"])
    assert O == pytest.approx(num["O"][0], abs=tol["O"])
    assert L == pytest.approx(num["L"][0], abs=tol["L"])


@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_blockwise_recurrence_equals_oracle(oracle_lib, block):
    """The merge rule the GPU kernels use (rescale-and-add over blocks) reaches
    the oracle's plain definition on random rows, for any block size."""
    rng = np.random.default_rng(block)
    n = 50
    s = rng.normal(0, 3, n).astype(np.float32)
    vals = rng.normal(0, 1, n).astype(np.float32)
    q, k, v = _score_encoding(s, values=vals)
    O, L = _decode_rows(oracle_lib, q, k, v, 1.0)
    sb = _bf16(s).float().numpy().astype(float)
    vb = _bf16(vals).float().numpy().astype(float)
    Ob, Lb, _ = _blockwise(sb, vb, block)
    assert O[0] == pytest.approx(Ob, abs=1e-12)
    assert L == pytest.approx(Lb, abs=1e-12)


# -------------------------------------------------------------- stress rows

def _stress_rows():
    return {k: [float(x) for x in v] for k, v in read_golden("softmax_stress_rows.txt").items()}


@pytest.mark.parametrize("name", list(_stress_rows()))
def test_stress_rows_are_distributions(oracle_lib, name):
    s = _stress_rows()[name]
    q, k, v = _score_encoding(s)
    Ow, L = _decode_rows(oracle_lib, q, k, v, 1.0, seed=len(s))
    w = Ow[:len(s)]
    assert np.all(np.isfinite(w)) and np.isfinite(L)
    assert abs(w.sum() - 1.0) <= 1e-12                 # the page's criterion is 0.01
    assert np.all(Ow[len(s):] == 0)
    sb = _bf16(s).float().numpy()
    # weights are ordered like the scores (a sign slip would reverse them)
    order = np.argsort(sb, kind="stable")
    assert np.all(np.diff(w[order]) >= -1e-15)
    # each weight equals exp(s_j - LSE) (the LSE is the log of the normaliser)
    np.testing.assert_allclose(w, np.exp(sb.astype(float) - L), rtol=1e-12, atol=1e-300)


def test_stress_tied_row_is_uniform(oracle_lib):
    s = _stress_rows()["tied_max_8"]
    q, k, v = _score_encoding(s)
    Ow, L = _decode_rows(oracle_lib, q, k, v, 1.0)
    np.testing.assert_allclose(Ow[:8], np.full(8, 1 / 8), rtol=0, atol=1e-15)
    assert L == pytest.approx(3.0 + math.log(8.0), abs=1e-12)


def test_stress_spike_dominates(oracle_lib):
    s = _stress_rows()["stability_spike_8"]
    q, k, v = _score_encoding(s)
    Ow, L = _decode_rows(oracle_lib, q, k, v, 1.0)
    assert Ow[3] == pytest.approx(1.0, abs=1e-20) and Ow[3] <= 1.0
    assert L == pytest.approx(50.0, abs=1e-18)


@pytest.mark.parametrize("shift", [-64.0, -3.5, 7.0, 100.0])
def test_score_shift_invariance(oracle_lib, shift):
    """Adding c to every score leaves the weights unchanged and adds c to LSE."""
    s = _stress_rows()["bigger_16"]
    q, k, v = _score_encoding(s)
    O0, L0 = _decode_rows(oracle_lib, q, k, v, 1.0)
    q2, k2, v2 = _score_encoding(s, shift=shift)
    O1, L1 = _decode_rows(oracle_lib, q2, k2, v2, 1.0, seed=9)
    np.testing.assert_allclose(O1, O0, rtol=1e-12, atol=1e-15)
    assert L1 == pytest.approx(L0 + shift, abs=1e-12)


# ------------------------------------------------------------- closed forms

def test_zero_query_gives_causal_running_mean(oracle_lib):
    """q = 0 makes every score 0: row t is the mean of V[0..t], LSE = ln(t+1)."""
    case = W.make_prefill("zq", B=2, T=37, Hq=8, Hkv=2, d=D, n_pages=32, seed=11,
                          seq_lens=[37, 21], n_layers=2, layer=1, fill_other_layers=True)
    case.q = torch.zeros_like(case.q)
    O, L, _ = oracle_lib.prefill_case(case)
    O = O.reshape(2, 37, 8, D)
    L = L.reshape(2, 37, 8)
    for b, n in enumerate(case.seq_lens):
        vb = case.tokens.v[case.tokens.slot_ids == case.slot_ids[b]].double().numpy()  # [n, Hkv, d]
        for t in range(37):
            if t >= n:
                assert np.all(O[b, t] == 0) and np.all(np.isneginf(L[b, t]))
                continue
            mean = vb[:t + 1].mean(axis=0)                     # [Hkv, d]
            np.testing.assert_allclose(O[b, t], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-14)
            np.testing.assert_allclose(L[b, t], math.log(t + 1), rtol=0, atol=1e-14)


def test_zero_query_decode_is_context_mean(oracle_lib):
    case = W.make_decode("zq", B=3, Hq=8, Hkv=2, d=D, n_pages=64, ctx_lens=[1, 17, 100], seed=2)
    case.q = torch.zeros_like(case.q)
    O, L, _ = oracle_lib.decode_case(case)
    allk = torch.cat([case.context.v, case.new_tokens.v])
    slots = np.concatenate([case.context.slot_ids, case.new_tokens.slot_ids])
    for b, c in enumerate(case.ctx_lens):
        vb = allk[torch.from_numpy(slots == b)].double().numpy()
        mean = vb.mean(axis=0)
        np.testing.assert_allclose(O[b], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[b], math.log(c), rtol=0, atol=1e-14)


def test_single_key_returns_its_value(oracle_lib):
    case = W.make_prefill("t1", B=1, T=1, Hq=4, Hkv=1, d=D, n_pages=4, seed=4)
    O, L, _ = oracle_lib.prefill_case(case)
    v0 = case.tokens.v[0, 0].double().numpy()
    k0 = case.tokens.k[0, 0].double().numpy()
    for h in range(4):
        assert np.array_equal(O[0, h], v0)
        qh = case.q[0, 0, h].double().numpy()
        assert L[0, h] == pytest.approx(case.scale * float(qh @ k0), abs=1e-12)


def test_gqa_uses_consecutive_groups(oracle_lib):
    """With V = +1 on kv head 0 and -1 on kv head 1, q heads 0-3 must read +1
    and 4-7 read -1 (consecutive grouping, not interleaved)."""
    case = W.make_prefill("gqa", B=1, T=20, Hq=8, Hkv=2, d=D, n_pages=8, seed=6)
    v = torch.ones_like(case.tokens.v)
    v[:, 1] = -1.0
    case.tokens.v = v
    O, _, _ = oracle_lib.prefill_case(case)
    assert np.all(O[:, :4] == 1.0) and np.all(O[:, 4:] == -1.0)


def test_empty_context_decode(oracle_lib):
    case = W.make_decode("empty", B=2, Hq=4, Hkv=1, d=D, n_pages=8, ctx_lens=[0, 5], seed=1)
    O, L, _ = oracle_lib.decode_case(case)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(O[1])) and np.all(np.isfinite(L[1]))


# --------------------------------------------------------------- brute force

def _brute(q, k, v, scale, causal, lens):
    """Direct softmax(scale Q K^T + mask) V per (b, h) with contiguous K/V."""
    q = q.double().numpy()
    k = k.double().numpy()
    v = v.double().numpy()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, T, Hq, d))
    L = np.full((B, T, Hq), -np.inf)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            S = scale * q[b, :n, h] @ k[b, :n, h // g].T               # [n, n]
            if causal:
                S = np.where(np.tril(np.ones((n, n), bool)), S, -np.inf)
            lse = logsumexp(S, axis=1)
            O[b, :n, h] = np.exp(S - lse[:, None]) @ v[b, :n, h // g]
            L[b, :n, h] = lse
    return O, L


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 4), (32, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_brute_force(oracle_lib, Hq, Hkv, causal):
    case = W.make_prefill("bf", B=3, T=40, Hq=Hq, Hkv=Hkv, d=D, n_pages=40, seed=Hq + Hkv,
                          seq_lens=[40, 17, 1], causal=causal, n_layers=3, layer=2, n_slots=5,
                          slot_ids=[4, 0, 2], fill_other_layers=True, mbps=4)
    O, L, _ = oracle_lib.prefill_case(case)
    # rebuild contiguous K/V [B, T, Hkv, d] straight from the generator's token rows
    k = torch.zeros(3, 40, Hkv, D, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    tb = case.tokens
    inv = {int(s): b for b, s in enumerate(case.slot_ids)}
    bidx = np.array([inv[int(s)] for s in tb.slot_ids])
    k[bidx, tb.positions] = tb.k
    v[bidx, tb.positions] = tb.v
    Ob, Lb = _brute(case.q, k, v, case.scale, causal, case.seq_lens)
    np.testing.assert_allclose(O.reshape(Ob.shape), Ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(L.reshape(Lb.shape)), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L.reshape(Lb.shape)[fin], Lb[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,H,causal", [(64, 4, True), (128, 2, False), (128, 2, True)])
def test_dense_matches_brute_force(oracle_lib, d, H, causal):
    case = W.make_dense("dbf", B=2, T=33, Hq=H, Hkv=H, d=d, causal=causal, seed=d)
    O, L = oracle_lib.dense_case(case)
    Ob, Lb = _brute(case.q, case.k, case.v, case.scale, causal, [33, 33])
    np.testing.assert_allclose(O.reshape(Ob.shape), Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L.reshape(Lb.shape), Lb, rtol=0, atol=1e-12)


def test_dense_rows_subset_matches_full(oracle_lib):
    case = W.make_dense("rows", B=2, T=50, Hq=4, Hkv=2, d=D, causal=True, seed=8)
    O, L = oracle_lib.dense_case(case)
    rows = np.array([[1, 49], [0, 0], [1, 7]], np.int32)
    Os, Ls = oracle_lib.dense_case(case, rows=rows)
    for i, (b, t) in enumerate(rows):
        assert np.array_equal(Os[i], O[b * 50 + t]) and np.array_equal(Ls[i], L[b * 50 + t])


def test_decode_matches_brute_force(oracle_lib):
    case = W.make_decode("dbf", B=4, Hq=8, Hkv=2, d=D, n_pages=64, ctx_lens=[1, 16, 17, 150],
                         seed=7, n_layers=2, layer=1, n_slots=6, slot_ids=[5, 1, 3, 0])
    O, L, _ = oracle_lib.decode_case(case)
    allk = torch.cat([case.context.k, case.new_tokens.k])
    allv = torch.cat([case.context.v, case.new_tokens.v])
    slots = np.concatenate([case.context.slot_ids, case.new_tokens.slot_ids])
    pos = np.concatenate([case.context.positions, case.new_tokens.positions])
    for b in range(4):
        sel = np.flatnonzero(slots == case.slot_ids[b])
        sel = sel[np.argsort(pos[sel])]
        kb = allk[sel].double().numpy()
        vb = allv[sel].double().numpy()
        for h in range(8):
            s = case.scale * kb[:, h // 4] @ case.q[b, h].double().numpy()
            lse = logsumexp(s)
            np.testing.assert_allclose(O[b, h], np.exp(s - lse) @ vb[:, h // 4], rtol=0, atol=1e-12)
            assert L[b, h] == pytest.approx(lse, abs=1e-12)


# ---------------------------------------------------------------- invariants

def test_page_permutation_invariance(oracle_lib):
    """Where the pages sit in the pool does not change the result (bitwise)."""
    a = W.make_prefill("pa", B=2, T=45, Hq=8, Hkv=2, d=D, n_pages=64, seed=21)
    b = W.make_prefill("pb", B=2, T=45, Hq=8, Hkv=2, d=D, n_pages=64, seed=21)
    rng = np.random.default_rng(99)
    perm = rng.permutation(64).astype(np.int32)
    b.cache.block_table = np.where(a.cache.block_table >= 0, perm[np.maximum(a.cache.block_table, 0)], -1)
    assert not np.array_equal(a.cache.block_table, b.cache.block_table)
    Oa, La, _ = oracle_lib.prefill_case(a)
    Ob, Lb, _ = oracle_lib.prefill_case(b)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


def test_gqa_equals_repeated_heads(oracle_lib):
    """GQA with group g equals MHA on K/V heads repeated g times (consecutively)."""
    c = W.make_dense("g", B=1, T=30, Hq=8, Hkv=2, d=D, causal=True, seed=3)
    O, L = oracle_lib.dense_case(c)
    c.k = c.k.repeat_interleave(4, dim=2)
    c.v = c.v.repeat_interleave(4, dim=2)
    O2, L2 = oracle_lib.dense_case(c)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_decode_equals_last_prefill_row(oracle_lib):
    p = W.make_prefill("p", B=1, T=70, Hq=8, Hkv=2, d=D, n_pages=16, seed=12)
    Op, Lp, pool = oracle_lib.prefill_case(p)
    c = p.cache
    Od, Ld, bad = oracle_lib.attn_decode(p.q[:, -1], pool, c.n_pages, c.block_table, c.layer,
                                         p.slot_ids, np.array([70], np.int32), c.n_kv_heads, p.scale)
    assert bad == 0
    assert np.array_equal(Od[0], Op[-1]) and np.array_equal(Ld[0], Lp[-1])


def test_paged_prefill_equals_dense(oracle_lib):
    p = W.make_prefill("p", B=2, T=33, Hq=8, Hkv=2, d=D, n_pages=16, seed=13)
    Op, Lp, _ = oracle_lib.prefill_case(p)
    k = p.tokens.k.reshape(2, 33, 2, D)
    v = p.tokens.v.reshape(2, 33, 2, D)
    Od, Ld = oracle_lib.attn_dense(p.q, k, v, p.scale, True)
    assert np.array_equal(Op, Od) and np.array_equal(Lp, Ld)


def test_lse_normalises_rows(oracle_lib):
    """sum_j exp(s_ij - LSE_i) = 1 with scores recomputed independently."""
    c = W.make_dense("n", B=1, T=25, Hq=2, Hkv=2, d=D, causal=True, seed=14)
    _, L = oracle_lib.dense_case(c)
    q = c.q.double().numpy()[0]
    k = c.k.double().numpy()[0]
    for h in range(2):
        S = c.scale * q[:, h] @ k[:, h].T
        for t in range(25):
            assert math.fsum(np.exp(S[t, :t + 1] - L[t, h])) == pytest.approx(1.0, abs=1e-13)


def test_invalid_pages_are_counted_and_skipped(oracle_lib):
    case = W.make_decode("bad", B=1, Hq=4, Hkv=1, d=D, n_pages=16, ctx_lens=[40], seed=5)
    O, L, pool = oracle_lib.decode_case(case)
    bt = case.cache.block_table.copy()
    bt[0, 0, 1] = -1                      # tokens 16..31 lose their page
    O2, L2, bad = oracle_lib.attn_decode(case.q, pool, 16, bt, 0, None, case.ctx_lens, 1, case.scale)
    assert bad == 16 * 4
    allk = torch.cat([case.context.k, case.new_tokens.k]).double().numpy()
    allv = torch.cat([case.context.v, case.new_tokens.v]).double().numpy()
    keep = np.r_[0:16, 32:40]
    for h in range(4):
        s = case.scale * allk[keep, 0] @ case.q[0, h].double().numpy()
        lse = logsumexp(s)
        np.testing.assert_allclose(O2[0, h], np.exp(s - lse) @ allv[keep, 0], atol=1e-12, rtol=0)
    bt[0, 0, 0] = 16                      # out of range of the 16-page pool
    _, _, bad = oracle_lib.attn_decode(case.q, pool, 16, bt, 0, None, case.ctx_lens, 1, case.scale)
    assert bad == 32 * 4


# ------------------------------------------------------------------- scatter

def test_page_geometry_matches_printed_constants(oracle_lib):
    g = {k: int(v[0]) for k, v in read_golden("page_geometry.txt").items()}
    assert g["kv_dim"] == W.LLAMA_HKV * W.LLAMA_D
    assert oracle_lib.page_bytes(W.LLAMA_HKV, W.LLAMA_D) == g["block_bytes"]
    assert g["block_bytes"] == 2 * g["v_offset_bytes"]
    assert g["v_offset_bytes"] == g["block_tokens"] * g["kv_dim"] * 2
    assert g["cache_bytes"] // oracle_lib.page_bytes(W.LLAMA_HKV, W.LLAMA_D) == g["num_blocks"]
    assert g["max_sequences"] * g["n_layers"] * g["max_blocks_per_seq"] == g["block_table_entries"]


@pytest.mark.parametrize("Hkv,d", [(8, 64), (2, 128)])
def test_scatter_places_rows_at_page_addresses(oracle_lib, Hkv, d):
    """Whole-pool check against a numpy view of the page as [K|V][token][head][dim]."""
    case = W.make_prefill("sc", B=3, T=50, Hq=Hkv, Hkv=Hkv, d=d, n_pages=30, seed=31,
                          seq_lens=[50, 3, 33], n_layers=2, layer=1, n_slots=4, slot_ids=[2, 3, 0])
    pool = oracle_lib.new_pool(30, Hkv, d, 0xBEEF)
    assert oracle_lib.scatter_tokens(pool, case.cache, case.tokens) == 0
    exp = np.full((30, 2, 16, Hkv, d), 0xBEEF, np.uint16)
    tb = case.tokens
    kb = tb.k.view(torch.int16).numpy().view(np.uint16)
    vb = tb.v.view(torch.int16).numpy().view(np.uint16)
    for i in range(len(tb.positions)):
        page = case.cache.block_table[tb.slot_ids[i], 1, tb.positions[i] // 16]
        exp[page, 0, tb.positions[i] % 16] = kb[i]
        exp[page, 1, tb.positions[i] % 16] = vb[i]
    assert np.array_equal(pool.view(np.uint16).reshape(exp.shape), exp)


def test_scatter_skips_invalid_entries(oracle_lib):
    case = W.make_prefill("sc", B=1, T=20, Hq=8, Hkv=8, d=D, n_pages=4, seed=1)
    bt = case.cache.block_table.copy()
    bt[0, 0, 1] = -1
    pool = oracle_lib.new_pool(4, 8, D, 0x1234)
    bad = oracle_lib.kv_scatter(pool, 4, case.tokens.k, case.tokens.v, case.tokens.slot_ids,
                                case.tokens.positions, bt, 0, 8, D)
    assert bad == 4
    words = pool.view(np.uint16).reshape(4, 2, 16, 8, D)
    untouched = [p for p in range(4) if p != bt[0, 0, 0]]
    assert np.all(words[untouched] == 0x1234)
