"""Pins of the oracle's decode-append part: bfloat16 rounding, RoPE, page
allocation from the free stack, page release.

Each pin takes a route of its own: rounding against brute force over the two
neighbouring bfloat16 values and against torch's fp32 -> bf16 cast; RoPE
against complex multiplication in numpy and against the rotation's
relative-position property; allocation and release against orders derived
by hand from the pages' pop/push rules (tiny-vllm part 6, "The lifetime of a
physical block: free_blocks"); the page writes against a numpy view of the
page layout.
"""

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_tensor(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ rounding

def test_round_bf16_brute_force(oracle_lib):
    """Nearest of the two bf16 neighbours, ties to the even pattern, for random doubles,
    exact halfway points, and values next to them."""
    rng = np.random.default_rng(5)
    mant = rng.integers(0, 1 << 16, size=4000).astype(np.uint32)
    base_bits = (rng.integers(0x0080, 0x7F00, size=4000).astype(np.uint32))
    lo = _bits_to_f64(base_bits.astype(np.uint16))
    hi = _bits_to_f64((base_bits + 1).astype(np.uint16))
    frac = mant / 65536.0
    x = lo + (hi - lo) * frac                                   # includes exact halves (mant=32768)
    x = np.concatenate([x, (lo + hi) / 2, np.nextafter((lo + hi) / 2, np.inf),
                        np.nextafter((lo + hi) / 2, -np.inf)])
    lo2 = np.concatenate([lo, lo, lo, lo]); hi2 = np.concatenate([hi, hi, hi, hi])
    b_lo = np.concatenate([base_bits] * 4)
    sign = rng.choice([-1.0, 1.0], size=x.shape)
    got = oracle_lib.round_bf16(sign * x)
    d_lo, d_hi = np.abs(x - lo2), np.abs(hi2 - x)
    want = np.where(d_lo < d_hi, b_lo, np.where(d_hi < d_lo, b_lo + 1, np.where(b_lo % 2 == 0, b_lo, b_lo + 1)))
    want = want.astype(np.uint16) | np.where(sign < 0, 0x8000, 0).astype(np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch_on_fp32_values(oracle_lib):
    """On values exact in fp32 the result is torch's round-to-nearest-even cast."""
    rng = np.random.default_rng(6)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    f = np.concatenate([f, np.float32([0.0, -0.0, 1e-40, -3e-39, 3.0e38, 65504.0])])
    want = _bits(torch.from_numpy(f).to(torch.bfloat16))
    assert np.array_equal(oracle_lib.round_bf16(f.astype(np.float64)), want)


# ---------------------------------------------------------------------- RoPE

def _rand_rows(seed, n, H, d):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(n, H, d, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_is_complex_rotation(oracle_lib, d):
    """Pair i = (x[i], x[i+d/2]) read as x[i] + j x[i+d/2], multiplied by cos + j sin."""
    x = _rand_rows(1, 5, 3, d)
    cos_t, sin_t = W.random_angle_tables(40, d, seed=2)
    pos = np.array([0, 7, 39, 16, 1], np.int32)
    y = oracle_lib.rope(x, pos, cos_t, sin_t)
    xf = x.float().numpy().astype(np.float64)
    z = xf[..., : d // 2] + 1j * xf[..., d // 2:]
    rot = cos_t[pos].astype(np.float64) + 1j * sin_t[pos].astype(np.float64)
    w = z * rot[:, None, :]
    assert np.allclose(y[..., : d // 2], w.real, rtol=0, atol=1e-12)
    assert np.allclose(y[..., d // 2:], w.imag, rtol=0, atol=1e-12)


def test_rope_special_angles(oracle_lib):
    """cos 1, sin 0 leaves x as it is; cos 0, sin 1 maps (a, b) to (-b, a); cos -1 negates."""
    d = 64
    x = _rand_rows(3, 1, 2, d)
    cos_t = np.array([[1.0] * 32, [0.0] * 32, [-1.0] * 32], np.float32)
    sin_t = np.array([[0.0] * 32, [1.0] * 32, [0.0] * 32], np.float32)
    xf = x.float().numpy().astype(np.float64)
    for p, want in [(0, xf), (1, np.concatenate([-xf[..., 32:], xf[..., :32]], -1)), (2, -xf)]:
        y = oracle_lib.rope(x, np.array([p], np.int32), cos_t, sin_t)
        assert np.array_equal(y, want)


def test_rope_relative_position(oracle_lib):
    """With angles pos * theta_i the dot product of rotated q at m and k at n depends on m - n only."""
    d = 64
    cos_t, sin_t = W.rope_tables(600, d)
    q, k = _rand_rows(4, 1, 1, d), _rand_rows(5, 1, 1, d)

    def dot(m, n):
        a = oracle_lib.rope(q, np.array([m], np.int32), cos_t, sin_t)
        b = oracle_lib.rope(k, np.array([n], np.int32), cos_t, sin_t)
        return float((a * b).sum())

    for m, n, shift in [(5, 3, 100), (40, 0, 411), (17, 17, 512)]:
        assert abs(dot(m, n) - dot(m + shift, n + shift)) < 2e-4
    assert abs(dot(9, 2) - dot(2, 9)) > 1e-3          # and it is not symmetric in m - n


def test_rope_bad_position_rows_are_nan(oracle_lib):
    x = _rand_rows(6, 3, 2, 64)
    cos_t, sin_t = W.rope_tables(8, 64)
    y = oracle_lib.rope(x, np.array([3, 8, -1], np.int32), cos_t, sin_t)
    assert np.isfinite(y[0]).all() and np.isnan(y[1]).all() and np.isnan(y[2]).all()


# ------------------------------------------------------- allocation + write

def _one_token_rows(B, Hkv, d, seed=11):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, d, generator=g).to(torch.bfloat16)
    return k, v


def test_append_pop_order_by_hand(oracle_lib):
    """Stack [10, 11, 12, 13] (top 4).  Tokens in batch order: slot 0 at position 16 opens block 1,
    slot 1 at 5 writes into its block 0, slot 2 at 0 opens block 0, slot 3 at 32 opens block 2.
    Popping from the back in batch order gives 13, 12, 11; one page (10) stays free."""
    Hkv, d, n_pages = 2, 64, 16
    bt = np.full((4, 1, 4), -1, np.int32)
    bt[0, 0, 0] = 3
    bt[1, 0, 0] = 4
    bt[3, 0, :2] = [5, 6]
    k, v = _one_token_rows(4, Hkv, d)
    cos_t, sin_t = W.rope_tables(64, d)
    pool = oracle_lib.new_pool(n_pages, Hkv, d, 0x1111)
    _, top, errs = oracle_lib.kv_append(pool, n_pages, k, v, np.array([16, 5, 0, 32], np.int32),
                                        cos_t, sin_t, bt, 0, np.array([10, 11, 12, 13], np.int32), 4)
    assert errs == 0 and top == 1
    want = np.full((4, 1, 4), -1, np.int32)
    want[0, 0, :2] = [3, 13]
    want[1, 0, 0] = 4
    want[2, 0, 0] = 12
    want[3, 0, :3] = [5, 6, 11]
    assert np.array_equal(bt, want)
    # rows land at (page, row pos % 16): K rotated, V as given; nothing else changes
    words = pool.view(np.uint16).reshape(n_pages, 2, 16, Hkv, d)
    kr = oracle_lib.round_bf16(oracle_lib.rope(k, np.array([16, 5, 0, 32], np.int32), cos_t, sin_t))
    vb = _bits(v)
    expect = np.full(words.shape, 0x1111, np.uint16)
    for b, (page, row) in enumerate([(13, 0), (4, 5), (12, 0), (11, 0)]):
        expect[page, 0, row] = kr[b]
        expect[page, 1, row] = vb[b]
    assert np.array_equal(words, expect)


def test_append_equals_rope_then_scatter(oracle_lib):
    """On a seeded decode state, the append equals: allocate by hand, RoPE + round the K rows,
    then the (separately pinned) scatter; the query comes back rotated and rounded."""
    case = W.make_append("ap", B=24, Hq=8, Hkv=2, d=64, n_pages=400, max_ctx=300, seed=3,
                         ctx_lens=[1, 17, 33, 16, 2, 300, 49, 64, 65, 97] + [5 + 11 * i for i in range(14)],
                         mbps=24, n_slots=30, slot_ids=np.arange(24)[::-1] + 3)
    dc = case.decode
    nt = dc.new_tokens
    # new_tokens are in batch order
    assert np.array_equal(nt.slot_ids, dc.slot_ids) and np.array_equal(nt.positions, dc.ctx_lens - 1)
    pool = oracle_lib.pool_for(dc)
    assert oracle_lib.scatter_tokens(pool, dc.cache, dc.context) == 0
    pool_ref = pool.copy()
    bt = case.block_table.copy()
    q_out, top, errs = oracle_lib.kv_append(pool, dc.cache.n_pages, nt.k, nt.v, nt.positions,
                                            case.cos_t, case.sin_t, bt, 0, case.free_pages, case.top,
                                            slot_ids=dc.slot_ids, q=dc.q)
    assert errs == 0
    # by hand: openers in batch order take the stack from the back
    bt_ref = case.block_table.copy()
    t = case.top
    for b in range(dc.B):
        p = int(nt.positions[b])
        if p % 16 == 0:
            t -= 1
            bt_ref[dc.slot_ids[b], 0, p // 16] = case.free_pages[t]
    assert top == t and np.array_equal(bt, bt_ref)
    kr = oracle_lib.round_bf16(oracle_lib.rope(nt.k, nt.positions, case.cos_t, case.sin_t))
    assert oracle_lib.kv_scatter(pool_ref, dc.cache.n_pages, kr, nt.v, nt.slot_ids, nt.positions,
                                 bt_ref, 0, 2, 64) == 0
    assert np.array_equal(pool, pool_ref)
    qr = oracle_lib.round_bf16(oracle_lib.rope(dc.q, nt.positions, case.cos_t, case.sin_t))
    assert np.array_equal(q_out, qr)


def test_append_runs_out_of_pages(oracle_lib):
    """Three openers, two free pages: the third opener finds the stack empty, its token is not
    written and its entry stays -1; the stack ends empty."""
    Hkv, d, n_pages = 1, 64, 8
    bt = np.full((3, 1, 2), -1, np.int32)
    k, v = _one_token_rows(3, Hkv, d)
    cos_t, sin_t = W.rope_tables(32, d)
    pool = oracle_lib.new_pool(n_pages, Hkv, d, 0x2222)
    _, top, errs = oracle_lib.kv_append(pool, n_pages, k, v, np.array([0, 16, 0], np.int32), cos_t,
                                        sin_t, bt, 0, np.array([6, 7], np.int32), 2)
    assert errs == oracle_lib.ERR_NO_FREE_PAGE and top == 0
    assert bt[0, 0, 0] == 7 and bt[1, 0, 1] == 6 and bt[2, 0, 0] == -1
    words = pool.view(np.uint16).reshape(n_pages, -1)
    assert np.all(words[[0, 1, 2, 3, 4, 5]] == 0x2222)


def test_append_flags(oracle_lib):
    """Duplicate slot, re-assigned entry, slot and position out of range, a -1 entry mid-block."""
    Hkv, d, n_pages = 1, 64, 8
    k, v = _one_token_rows(5, Hkv, d)
    cos_t, sin_t = W.rope_tables(32, d)
    bt = np.full((4, 1, 2), -1, np.int32)
    bt[0, 0, 0] = 2                                   # slot 0 opens block 0 again: re-assigned
    pool = oracle_lib.new_pool(n_pages, Hkv, d, 0)
    _, top, errs = oracle_lib.kv_append(pool, n_pages, k[:2], v[:2], np.array([0, 3], np.int32),
                                        cos_t, sin_t, bt, 0, np.array([5], np.int32), 1,
                                        slot_ids=np.array([0, 1], np.int32))
    assert errs == oracle_lib.ERR_REASSIGNED | oracle_lib.ERR_BAD_PAGE and top == 0
    assert bt[0, 0, 0] == 5
    bt = np.full((4, 1, 2), -1, np.int32)
    _, top, errs = oracle_lib.kv_append(pool, n_pages, k[:4], v[:4], np.array([0, 0, 40, 0], np.int32),
                                        cos_t, sin_t, bt, 0, np.array([4, 5, 6], np.int32), 3,
                                        slot_ids=np.array([1, 1, 2, 9], np.int32))
    # slot 1 twice: both open its block 0, so the second one also re-assigns the entry
    assert errs == (oracle_lib.ERR_DUP_SLOT | oracle_lib.ERR_REASSIGNED | oracle_lib.ERR_BAD_POS
                    | oracle_lib.ERR_BAD_SLOT)
    assert top == 1 and bt[1, 0, 0] == 5              # the two valid openers popped 6 then 5


# ------------------------------------------------------------------- release

def test_release_push_order_by_hand(oracle_lib):
    """Release slots [2, 0] of a 2-layer table: slot 2 layer 0 blocks ascending, then layer 1,
    then slot 0; entries become -1; the untouched slot keeps its pages."""
    bt = np.full((3, 2, 3), -1, np.int32)
    bt[2, 0] = [7, -1, 4]
    bt[2, 1] = [-1, 9, 1]
    bt[0, 1] = [3, 8, -1]
    bt[1, 0] = [5, 6, 0]
    stack = np.full(10, -7, np.int32)
    stack[:2] = [2, 11]
    top, errs = oracle_lib.kv_release(np.array([2, 0], np.int32), bt, stack, 2)
    assert errs == 0 and top == 8
    assert list(stack[:8]) == [2, 11, 7, 4, 9, 1, 3, 8] and list(stack[8:]) == [-7, -7]
    assert np.all(bt[[0, 2]] == -1) and list(bt[1, 0]) == [5, 6, 0]


def test_release_stack_full_and_bad_slot(oracle_lib):
    bt = np.full((2, 1, 4), -1, np.int32)
    bt[0, 0] = [1, 2, 3, 4]
    stack = np.zeros(3, np.int32)
    top, errs = oracle_lib.kv_release(np.array([5, 0], np.int32), bt, stack, 1)
    assert errs == oracle_lib.ERR_BAD_SLOT | oracle_lib.ERR_STACK_FULL and top == 3
    assert list(stack) == [0, 1, 2] and list(bt[0, 0]) == [-1, -1, 3, 4]


def test_append_release_round_trip(oracle_lib):
    """Appending 40 tokens to a fresh slot takes 3 pages from the stack; releasing the slot puts
    the same 3 pages back, so the free set is what it was."""
    Hkv, d, n_pages = 1, 64, 12
    cos_t, sin_t = W.rope_tables(64, d)
    bt = np.full((2, 1, 4), -1, np.int32)
    stack = np.arange(n_pages, dtype=np.int32)[::-1].copy()
    top = n_pages
    pool = oracle_lib.new_pool(n_pages, Hkv, d, 0)
    k, v = _one_token_rows(40, Hkv, d)
    for p in range(40):
        _, top, errs = oracle_lib.kv_append(pool, n_pages, k[p:p + 1], v[p:p + 1],
                                            np.array([p], np.int32), cos_t, sin_t, bt, 0, stack, top,
                                            slot_ids=np.array([1], np.int32))
        assert errs == 0
    assert top == n_pages - 3 and sorted(bt[1, 0, :3]) == [0, 1, 2]
    top, errs = oracle_lib.kv_release(np.array([1], np.int32), bt, stack, top)
    assert errs == 0 and top == n_pages and sorted(stack) == list(range(n_pages))
