"""Helpers shared by the GPU parity tests: move seeded cases to the device,
run the library through its binding, and compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_amd as pa

DEV = torch.device("cuda")
O_TOL = 2e-2        # max |dO| for the bf16 output
LSE_TOL = 1e-3      # max |dLSE|


def i32(x) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def device_pool(cache) -> torch.Tensor:
    """Device pool (uint8) filled with the case's bf16 fill pattern."""
    fill = cache.page_fill if cache.page_fill < 0x8000 else cache.page_fill - 0x10000
    words = torch.full((cache.pool_bytes // 2,), fill, dtype=torch.int16, device=DEV)
    return words.view(torch.uint8)


def scatter(pool: torch.Tensor, cache, tokens, bt: torch.Tensor | None = None,
            err: torch.Tensor | None = None) -> None:
    if len(tokens.positions) == 0:
        return
    pa.kv_scatter(tokens.k.to(DEV), tokens.v.to(DEV), i32(tokens.slot_ids), i32(tokens.positions),
                  pool, i32(cache.block_table) if bt is None else bt, cache.layer, err=err)


def run_prefill(case, pool: torch.Tensor | None = None, err: torch.Tensor | None = None):
    """Scatter (unless a pool is given) then prefill on the GPU; returns (O, LSE, pool) on device."""
    c = case.cache
    bt = i32(c.block_table)
    if pool is None:
        pool = device_pool(c)
        scatter(pool, c, case.tokens, bt)
    q_lens = getattr(case, "q_lens", None)
    O, L = pa.attn_prefill(case.q.to(DEV), pool, bt, c.layer, i32(case.seq_lens), c.n_kv_heads,
                           case.scale, case.causal, slot_ids=i32(case.slot_ids), err=err,
                           q_lens=None if q_lens is None else i32(q_lens))
    return O, L, pool


def run_decode(case, pool: torch.Tensor | None = None, err: torch.Tensor | None = None):
    c = case.cache
    bt = i32(c.block_table)
    if pool is None:
        pool = device_pool(c)
        scatter(pool, c, case.context, bt)
        scatter(pool, c, case.new_tokens, bt)
    O, L = pa.attn_decode(case.q.to(DEV), pool, bt, c.layer, i32(case.ctx_lens), c.n_kv_heads,
                          case.scale, max(case.max_ctx, 1), slot_ids=i32(case.slot_ids), err=err)
    return O, L, pool


def assert_attn_close(O_gpu: torch.Tensor, L_gpu: torch.Tensor, O_ref: np.ndarray,
                      L_ref: np.ndarray, o_tol: float = O_TOL, lse_tol: float = LSE_TOL,
                      what: str = "") -> None:
    """Element-wise check: O within o_tol, LSE within lse_tol (-inf must match -inf)."""
    Og = O_gpu.float().cpu().numpy().astype(np.float64).reshape(O_ref.shape)
    Lg = L_gpu.float().cpu().numpy().astype(np.float64).reshape(L_ref.shape)
    assert np.all(np.isfinite(Og)), f"{what}: non-finite O"
    dO = np.abs(Og - O_ref)
    i = np.unravel_index(np.argmax(dO), dO.shape)
    assert dO.max() <= o_tol, f"{what}: max|dO| = {dO.max():.3e} at {i} (gpu {Og[i]}, ref {O_ref[i]})"
    ninf_ref = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(Lg), ninf_ref), f"{what}: -inf LSE pattern differs"
    if (~ninf_ref).any():
        dL = np.abs(Lg[~ninf_ref] - L_ref[~ninf_ref])
        assert dL.max() <= lse_tol, f"{what}: max|dLSE| = {dL.max():.3e}"


def prefill_rows_layout(O_gpu: torch.Tensor, L_gpu: torch.Tensor, rows: np.ndarray):
    """Gather GPU rows (b, t) into the oracle's [n_rows, Hq, d] / [n_rows, Hq] layout."""
    b = torch.as_tensor(rows[:, 0], device=O_gpu.device, dtype=torch.long)
    t = torch.as_tensor(rows[:, 1], device=O_gpu.device, dtype=torch.long)
    return O_gpu[b, t], L_gpu[b, :, t]


def sample_rows(B: int, T: int, per_seq: int, seed: int = 0) -> np.ndarray:
    """(b, t) rows: first, last, tile edges and seeded random rows of each sequence."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        fixed = {0, 1, 31, 32, 63, 64, T // 2, T - 2, T - 1}
        ts = sorted({t for t in fixed if 0 <= t < T} | set(rng.integers(0, T, per_seq).tolist()))
        rows += [(b, t) for t in ts]
    return np.array(rows, np.int32)
