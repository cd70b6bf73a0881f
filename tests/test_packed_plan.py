"""attn_prefill_packed_plan on the host (no GPU): the work list covers every row
block's visible key tiles exactly once, split row blocks get distinct partial
slots and one merge item each, items come longest first, and bad arguments are
rejected.  The library assumes 256 CUs where no GPU is present."""

import ctypes

import numpy as np
import pytest

import paged_kv_cache_amd as pa


def plan(q_lens, kv_lens, Hq=32, Hkv=8, d=64, causal=True):
    p = pa.prefill_packed_plan(q_lens, kv_lens, Hq, Hkv, d, causal, device="cpu")
    items = p.host[:6 * p.n_work].reshape(-1, 6)
    merges = p.host[6 * p.n_work:6 * (p.n_work + p.n_merge)].reshape(-1, 6)
    return p, items, merges


def row_blocks(q_lens, kv_lens, Hq, Hkv, causal):
    """Every (b, rb, hg) with visible keys and its key-tile count, by the
    definition: BM = 32 * 4 / min(G, 4) rows of min(G, 4) heads; row t of
    sequence b sees keys 0 .. kv - q + t (causal) or all kv."""
    G = Hq // Hkv
    HW = min(G, 4)
    BM = 32 * 4 // HW
    out = {}
    for b, (q, kv) in enumerate(zip(q_lens, kv_lens)):
        for rb in range((q + BM - 1) // BM):
            last = min((rb + 1) * BM, q) - 1
            keys = (kv - q + last + 1) if causal else kv
            for hg in range(Hq // HW):
                out[(b, rb, hg)] = -(-keys // 64)
    return out, BM * HW


def dealt_model(items, n_hgroups):
    """The order the planner promises, rebuilt from its items: (sequence, head
    group) groups dealt largest first (by key tiles) to the least loaded of 8
    XCDs, each XCD's items longest first (ties in sequence order), then position
    i taken from XCD i % 8, or, once that list is empty, from the longest list.
    Within each XCD's list every other layer of 32 items (one per CU) is
    reversed."""
    base = sorted((tuple(x) for x in items), key=lambda x: (x[0], x[1], x[2], x[3]))
    tiles = {}
    for b, rb, hg, t0, t1, s in base:
        tiles[(b, hg)] = tiles.get((b, hg), 0) + (t1 - t0)
    groups = sorted(tiles, key=lambda g: (-tiles[g], g[0] * n_hgroups + g[1]))
    load, xcd = [0] * 8, {}
    for g in groups:
        x = load.index(min(load))
        xcd[g] = x
        load[x] += tiles[g]
    per = [[] for _ in range(8)]
    for it in base:
        per[xcd[(it[0], it[2])]].append(it)
    per = [sorted(v, key=lambda x: -(x[4] - x[3])) for v in per]
    layer = 256 // 8                     # the CUs of one XCD (256 CUs assumed without a GPU)
    for v in per:                        # every other layer reversed
        for l0 in range(layer, len(v), 2 * layer):
            v[l0:l0 + layer] = v[l0:l0 + layer][::-1]
    out = []
    for i in range(len(base)):
        x = i % 8
        if not per[x]:
            x = max(range(8), key=lambda y: (len(per[y]), -y))
        out.append(per[x].pop(0))
    return out


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 64), (16, 8, 128), (8, 8, 64), (8, 1, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_plan_covers_every_key_tile_once(Hq, Hkv, d, causal):
    rng = np.random.default_rng(Hq + d)
    ql = np.concatenate([[512, 300, 0, 64], np.ones(40, np.int64)])
    kv = np.concatenate([[1512, 9300, 20, 64], rng.integers(1, 5000, 40)])
    p, items, merges = plan(ql, kv, Hq, Hkv, d, causal)
    blocks, pairs = row_blocks(ql, kv, Hq, Hkv, causal)
    seen = {}
    for b, rb, hg, t0, t1, slot in items:
        assert 0 <= t0 < t1
        seen.setdefault((b, rb, hg), []).append((t0, t1, slot))
    assert set(seen) == set(blocks)
    slots = []
    merged = {(m[0], m[1], m[2]): (m[3], m[4]) for m in merges}
    assert len(merged) == len(merges)
    for key, parts in seen.items():
        parts.sort()
        assert parts[0][0] == 0 and parts[-1][1] == blocks[key]
        assert all(parts[i][1] == parts[i + 1][0] for i in range(len(parts) - 1))
        if len(parts) == 1:
            assert parts[0][2] == -1 and key not in merged
        else:
            first, n = merged[key]
            assert n == len(parts) and [s for _, _, s in parts] == list(range(first, first + n))
            slots += [s for _, _, s in parts]
    assert sorted(slots) == list(range(len(slots)))
    assert p.workspace_bytes == len(slots) * pairs * (d + 1) * 4
    # the order: one XCD (workgroup id mod 8) per (sequence, head group), each
    # XCD's items longest first -- checked against a model of the dealing
    assert [tuple(x) for x in items] == [tuple(x) for x in dealt_model(items, Hq // min(Hq // Hkv, 4))]


def test_plan_splits_only_long_row_blocks():
    # a small batch: nothing long enough to split, no workspace
    p, items, merges = plan([37, 1, 64], [300, 17, 64])
    assert p.n_merge == 0 and p.workspace_bytes == 0 and np.all(items[:, 5] == -1)
    # a chunk after a long prefix next to short work: its row blocks are cut into
    # pieces of at most the even share of key tiles per CU (256 CUs), >= 8 tiles,
    # halved while the plan has fewer than two items per CU
    ql, kv = [300, 1, 1], [13300, 5, 9]
    p, items, merges = plan(ql, kv)
    blocks, _ = row_blocks(ql, kv, 32, 8, True)
    # the decode rows are narrow row blocks (one row of 4 heads fits one wave):
    # they count a quarter of their key tiles; the rest count whole
    total = sum(n for (b, rb, hg), n in blocks.items() if b == 0) + sum(
        n for (b, rb, hg), n in blocks.items() if b > 0) // 4
    share = max(8, -(-total // 256))
    # fewer than two items per CU: the share is halved (not below 8) until there are
    while sum(-(-n // share) for n in blocks.values()) < 2 * 256 and share > 8:
        share = max(8, -(-share // 2))
    lengths = items[:, 4] - items[:, 3]
    assert p.n_merge > 0 and lengths.max() <= share
    for (b, rb, hg), n in blocks.items():
        k = (items[:, 0] == b) & (items[:, 1] == rb) & (items[:, 2] == hg)
        assert k.sum() == -(-n // share)
    # a batch whose row blocks are all shorter than the share is not split
    p, items, merges = plan([2048, 2048], [4096, 4096])
    assert p.n_work == 1024 and p.n_merge == 0


def test_plan_host_checks():
    lib = pa.load()
    nw, nm, wb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    ql = np.array([10, 1], np.int32)
    kv = np.array([100, 50], np.int32)
    args = lambda q, k: (q.ctypes.data, k.ctypes.data, 2, 32, 8, 64, 1)
    refs = (ctypes.byref(nw), ctypes.byref(nm), ctypes.byref(wb))
    assert lib.attn_prefill_packed_plan(*args(ql, kv), None, 0, *refs) == 0
    assert nw.value == 8 * 2 and nm.value == 0
    # a plan buffer too small: counts set, PA_ERR_WORKSPACE
    small = np.zeros(6, np.int32)
    assert lib.attn_prefill_packed_plan(*args(ql, kv), small.ctypes.data, 6, *refs) == -5
    assert nw.value == 16
    # q_len > kv_len, negative q_len
    assert lib.attn_prefill_packed_plan(*args(np.array([10, 60], np.int32), kv), None, 0, *refs) == -2
    assert lib.attn_prefill_packed_plan(*args(np.array([-1, 1], np.int32), kv), None, 0, *refs) == -2
    # unsupported head group, missing outputs, empty batch
    assert lib.attn_prefill_packed_plan(ql.ctypes.data, kv.ctypes.data, 2, 64, 2, 64, 1, None, 0, *refs) == -3
    assert lib.attn_prefill_packed_plan(ql.ctypes.data, kv.ctypes.data, 2, 32, 8, 64, 1, None, 0, None, None,
                                        None) == -1
    assert lib.attn_prefill_packed_plan(None, None, 0, 32, 8, 64, 1, None, 0, *refs) == 0


def test_packed_run_host_checks():
    lib = pa.load()
    g = ctypes.c_void_p(0x10000)
    base = [g, g, 64, g, 1, 1, 128, 0, None, g, g, 2, 100, 32, 8, 64, 0.125, 1, g, 16, 0, None, 0, g, g,
            None, None]
    # (every call below is rejected on the host or does nothing: none launches)
    bad = list(base)
    bad[16] = 0.0
    assert lib.attn_prefill_packed(*bad) == -8           # scale
    bad = list(base)
    bad[18] = None
    assert lib.attn_prefill_packed(*bad) == -1           # plan
    bad = list(base)
    bad[20] = 3                                          # merge items without a workspace
    assert lib.attn_prefill_packed(*bad) == -1
    bad = list(base)
    bad[0] = ctypes.c_void_p(0x10002)
    assert lib.attn_prefill_packed(*bad) == -4
    bad = list(base)
    bad[14] = 3
    assert lib.attn_prefill_packed(*bad) == -2           # Hq not a multiple of Hkv
    bad = list(base)
    bad[19] = 0
    assert lib.attn_prefill_packed(*bad) == 0            # no work: a no-op
