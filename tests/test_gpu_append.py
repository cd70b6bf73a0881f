"""kv_append and kv_release on the GPU against the oracle: pool bytes, block
table, free stack, allocator state, rotated query and error bits, all bit for
bit (the rotation is computed in fp64 and rounded once to bf16 on both sides)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _f32(x) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, np.float32))).to(DEV)


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DevState:
    """Device copy of an append case's cache state."""

    def __init__(self, case: W.AppendCase, stack_extra: int = 0):
        dc = case.decode
        self.cache = dc.cache
        self.pool = device_pool(dc.cache)
        self.bt = i32(case.block_table)
        cap = case.top + stack_extra
        fp = np.full(cap, -9, np.int32)
        fp[:case.top] = case.free_pages
        self.free = i32(fp)
        self.alloc = pa.new_alloc_state(case.top)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.cos, self.sin = _f32(case.cos_t), _f32(case.sin_t)
        if len(dc.context.positions):
            pa.kv_scatter(dc.context.k.to(DEV), dc.context.v.to(DEV), i32(dc.context.slot_ids),
                          i32(dc.context.positions), self.pool, i32(dc.cache.block_table),
                          dc.cache.layer)

    def append(self, k, v, positions, slot_ids, q=None):
        return pa.kv_append(k.to(DEV), v.to(DEV), i32(positions), self.cos, self.sin, self.pool,
                            self.bt, self.cache.layer, self.free, self.alloc,
                            slot_ids=None if slot_ids is None else i32(slot_ids),
                            q=None if q is None else q.to(DEV), err=self.err)


class HostState:
    """The oracle's copy of the same state."""

    def __init__(self, case: W.AppendCase):
        dc = case.decode
        self.cache = dc.cache
        self.pool = oracle.pool_for(dc)
        assert oracle.scatter_tokens(self.pool, dc.cache, dc.context) == 0
        self.bt = case.block_table.copy()
        self.free = case.free_pages.copy()
        self.top = case.top
        self.errs = 0
        self.case = case

    def append(self, k, v, positions, slot_ids, q=None):
        q_out, self.top, e = oracle.kv_append(self.pool, self.cache.n_pages, k, v, positions,
                                              self.case.cos_t, self.case.sin_t, self.bt,
                                              self.cache.layer, self.free, self.top,
                                              slot_ids=slot_ids, q=q)
        self.errs |= e
        return q_out


def _assert_same_state(dev: DevState, host: HostState, check_pool=True):
    torch.cuda.synchronize()
    assert int(dev.err.item()) == host.errs, f"err bits {int(dev.err.item())} vs {host.errs}"
    alloc = dev.alloc.cpu().numpy()
    assert int(alloc[0]) == host.top and int(alloc[1]) == 0
    bt = dev.bt.cpu().numpy()
    diff = np.argwhere(bt != host.bt)
    assert diff.size == 0, f"block table differs at {diff[:4].tolist()}"
    if check_pool:
        got = dev.pool.cpu().numpy()
        bad = np.flatnonzero(got != host.pool)
        assert bad.size == 0, f"{bad.size} pool bytes differ, first at {bad[:4]}"


def _one_step(case, check_pool=True):
    dc = case.decode
    nt = dc.new_tokens
    dev, host = DevState(case), HostState(case)
    qg = dev.append(nt.k, nt.v, nt.positions, dc.slot_ids, q=dc.q)
    qh = host.append(nt.k, nt.v, nt.positions, dc.slot_ids, q=dc.q)
    _assert_same_state(dev, host, check_pool)
    assert np.array_equal(_u16(qg), qh)
    return dev, host, qg, qh


def test_append_llama_batch_full_pool():
    """The 64-sequence decode batch (context U[1, 2048]) on the 2 GiB pool."""
    _one_step(W.llama_append())


@pytest.mark.parametrize("Hq,Hkv,d,random_angles", [(32, 8, 64, False), (8, 2, 64, True),
                                                    (16, 1, 128, True), (32, 8, 128, False)])
def test_append_ragged(Hq, Hkv, d, random_angles):
    # positions 0, 15, 16, 31, 32, ... : openers and non-openers, first and last rows of pages
    ctx = [1, 16, 17, 32, 33, 2, 48, 49, 64, 100, 113, 129, 255, 257, 1, 97]
    n = len(ctx)
    case = W.make_append("ragged", B=n, Hq=Hq, Hkv=Hkv, d=d, n_pages=300, ctx_lens=ctx, seed=d + Hq,
                         mbps=20, n_layers=3, layer=2, n_slots=n + 4,
                         slot_ids=np.random.default_rng(7).permutation(n + 4)[:n],
                         random_angles=random_angles, page_fill=0x7FC1)
    _one_step(case)


def test_append_many_steps_then_release():
    """Forty decode steps in a row for 12 sequences (pages opened along the way), then the
    release of 5 of them: state equal to the oracle's after every step."""
    case = W.make_append("steps", B=12, Hq=8, Hkv=2, d=64, n_pages=160, seed=9, mbps=16,
                         ctx_lens=[1, 5, 16, 17, 30, 31, 32, 60, 100, 3, 15, 47], n_slots=14,
                         slot_ids=[13, 0, 5, 7, 2, 9, 11, 1, 3, 8, 12, 4])
    dc = case.decode
    dev, host = DevState(case), HostState(case)
    g = torch.Generator().manual_seed(3)
    pos = dc.ctx_lens.astype(np.int32) - 1
    for step in range(40):
        k = torch.randn(12, 2, 64, generator=g).to(torch.bfloat16)
        v = torch.randn(12, 2, 64, generator=g).to(torch.bfloat16)
        q = torch.randn(12, 8, 64, generator=g).to(torch.bfloat16)
        qg = dev.append(k, v, pos, dc.slot_ids, q=q)
        qh = host.append(k, v, pos, dc.slot_ids, q=q)
        torch.cuda.synchronize()
        assert np.array_equal(_u16(qg), qh), f"step {step}: rotated query differs"
        _assert_same_state(dev, host, check_pool=(step % 10 == 9))
        pos = pos + 1
    rel = np.array([0, 9, 2, 13, 4], np.int32)
    pa.kv_release(i32(rel), dev.bt, dev.free, dev.alloc, err=dev.err)
    host.top, e = oracle.kv_release(rel, host.bt, host.free, host.top)
    host.errs |= e
    _assert_same_state(dev, host, check_pool=False)
    top = host.top
    assert np.array_equal(dev.free.cpu().numpy()[:top], host.free[:top])


def test_append_then_decode_matches_oracle():
    """The rotated query and the appended row feed attn_decode: same result as the oracle's
    append followed by its decode (tolerances of the attention parity)."""
    case = W.make_append("e2e", B=20, Hq=32, Hkv=8, d=64, n_pages=400, max_ctx=300, seed=12, mbps=20)
    dc = case.decode
    dev, host, qg, qh = _one_step(case)
    O, L = pa.attn_decode(qg, dev.pool, dev.bt, 0, i32(dc.ctx_lens), 8, dc.scale, int(dc.ctx_lens.max()))
    qh_t = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16)
    Oref, Lref, bad = oracle.attn_decode(qh_t, host.pool, dc.cache.n_pages, host.bt, 0, None,
                                         dc.ctx_lens, 8, dc.scale)
    assert bad == 0
    assert_attn_close(O, L, Oref, Lref, what="append+decode")


def test_append_runs_out_of_pages():
    """A stack of 3 pages for 7 opening tokens: four are flagged and left out, top ends at 0."""
    case = W.make_append("oop", B=10, Hq=8, Hkv=2, d=64, n_pages=64, seed=5, mbps=8,
                         ctx_lens=[1, 17, 33, 2, 49, 65, 3, 81, 97, 4])
    case.free_pages = case.free_pages[:3]
    dc = case.decode
    dev, host = DevState(case), HostState(case)
    dev.append(dc.new_tokens.k, dc.new_tokens.v, dc.new_tokens.positions, dc.slot_ids, q=dc.q)
    host.append(dc.new_tokens.k, dc.new_tokens.v, dc.new_tokens.positions, dc.slot_ids, q=dc.q)
    assert host.errs == oracle.ERR_NO_FREE_PAGE and host.top == 0
    _assert_same_state(dev, host)


def test_append_flags_bad_slot_position_and_reassigned():
    case = W.make_append("flags", B=6, Hq=8, Hkv=2, d=64, n_pages=64, seed=6, mbps=8,
                         ctx_lens=[17, 5, 33, 20, 1, 9], n_slots=8)
    dc = case.decode
    pos = dc.new_tokens.positions.copy()
    slots = dc.slot_ids.copy()
    slots[1] = 11                      # slot out of range
    pos[3] = 8 * 16 + 3                # beyond the table (rows of the tables reach 128)
    case.block_table[slots[0], 0, pos[0] // 16] = 63      # an opened block that already has a page
    dev, host = DevState(case), HostState(case)
    dev.append(dc.new_tokens.k, dc.new_tokens.v, pos, slots, q=dc.q)
    host.append(dc.new_tokens.k, dc.new_tokens.v, pos, slots, q=dc.q)
    assert host.errs == oracle.ERR_BAD_SLOT | oracle.ERR_BAD_POS | oracle.ERR_REASSIGNED
    _assert_same_state(dev, host)


def test_append_flags_duplicate_slot():
    """Two tokens naming one slot race on their writes; the flag is what is checked."""
    case = W.make_append("dup", B=4, Hq=8, Hkv=2, d=64, n_pages=64, seed=8, mbps=8,
                         ctx_lens=[5, 9, 13, 21])
    dc = case.decode
    dev = DevState(case)
    dev.append(dc.new_tokens.k, dc.new_tokens.v, dc.new_tokens.positions, np.array([0, 1, 1, 3], np.int32))
    torch.cuda.synchronize()
    assert int(dev.err.item()) == pa.PA_DEVERR_DUP_SLOT


def test_release_stack_full():
    case = W.make_append("rel", B=4, Hq=8, Hkv=2, d=64, n_pages=64, seed=10, mbps=8,
                         ctx_lens=[40, 70, 9, 100], n_layers=2)
    # free stack with room for 5 more pages only
    dev = DevState(case, stack_extra=5)
    host_bt = case.block_table.copy()
    host_free = np.full(case.top + 5, -9, np.int32)
    host_free[:case.top] = case.free_pages
    rel = np.array([3, 1], np.int32)
    pa.kv_release(i32(rel), dev.bt, dev.free, dev.alloc, err=dev.err)
    top, e = oracle.kv_release(rel, host_bt, host_free, case.top)
    torch.cuda.synchronize()
    assert e == oracle.ERR_STACK_FULL and int(dev.err.item()) == e
    assert int(dev.alloc[0].item()) == top == case.top + 5
    assert np.array_equal(dev.bt.cpu().numpy(), host_bt)
    assert np.array_equal(dev.free.cpu().numpy(), host_free)


def test_append_in_graph_carries_state_across_replays():
    """One decode step (append, then positions += 1) captured in a HIP graph and replayed 20
    times, with eager work and synchronisation between replays: same state as 20 oracle steps."""
    case = W.make_append("graph", B=16, Hq=8, Hkv=2, d=64, n_pages=200, seed=13, mbps=16,
                         ctx_lens=[1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 90, 120])
    dc = case.decode
    dev, host = DevState(case), HostState(case)
    k, v, q = dc.new_tokens.k.to(DEV), dc.new_tokens.v.to(DEV), dc.q.to(DEV)
    pos_d = i32(dc.new_tokens.positions)
    slots_d = i32(dc.slot_ids)
    q_out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        pa.kv_append(k, v, pos_d, dev.cos, dev.sin, dev.pool, dev.bt, 0, dev.free, dev.alloc,
                     slot_ids=slots_d, q=q, q_out=q_out, err=dev.err)
        pos_d.add_(1)
    pos = dc.new_tokens.positions.copy()
    for step in range(20):
        graph.replay()
        qh = host.append(dc.new_tokens.k, dc.new_tokens.v, pos, dc.slot_ids, q=dc.q)
        torch.cuda.synchronize()
        _ = (q_out.float() * 2).sum().item()           # eager work between replays
        assert np.array_equal(_u16(q_out), qh), f"replay {step}: rotated query differs"
        pos = pos + 1
    _assert_same_state(dev, host)
