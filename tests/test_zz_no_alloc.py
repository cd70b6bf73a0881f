"""attn_decode_noalloc (the no-allocation decode entry point) through the C ABI:
two calls in a row on one GPU, the second with a smaller input, each equal bit
for bit to attn_decode with a caller workspace (same kernels, same splits) and
within the attention tolerance of the oracle.  The first call fills the
library's static array with the partials of 4 x 16384 contexts; the second
(fewer, shorter contexts) must not see any of them."""

import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, device_pool, i32, scatter

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _both(case):
    c = case.cache
    pool = device_pool(c)
    bt = i32(c.block_table)
    scatter(pool, c, case.context, bt)
    scatter(pool, c, case.new_tokens, bt)
    q, lens, sid = case.q.to(DEV), i32(case.ctx_lens), i32(case.slot_ids)
    O_ws, L_ws = pa.attn_decode(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, case.max_ctx,
                                slot_ids=sid)
    O = torch.full_like(q, float("nan"))
    L = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.attn_decode_noalloc(q, pool, bt, c.layer, lens, c.n_kv_heads, case.scale, case.max_ctx, O, L,
                           slot_ids=sid, err=err)
    torch.cuda.synchronize()
    return O_ws, L_ws, O, L, int(err.item())


def test_noalloc_equals_workspace_decode_twice():
    big = W.long_decode()
    small = W.make_decode("small", B=2, Hq=32, Hkv=8, d=64, n_pages=512, ctx_lens=[3000, 700], seed=9)
    # the array is used: partials of the whole-page path (or of split contexts)
    assert pa.decode_workspace_size(big.B, big.Hq, 8, big.d, big.max_ctx) > 0
    assert pa.decode_workspace_size(small.B, small.Hq, 8, small.d, small.max_ctx) > 0
    for case in (big, small):
        O_ws, L_ws, O, L, err = _both(case)
        assert err == 0
        assert torch.equal(O, O_ws) and torch.equal(L, L_ws), case.name
        Oref, Lref, _ = oracle.decode_case(case)
        assert_attn_close(O, L, Oref, Lref, what=case.name)
