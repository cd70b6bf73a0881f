"""Python binding of libpagedattn.so (MI355X / gfx950 paged causal GQA attention).

Argument marshalling only: every step of the path runs in the library's HIP
kernels, launched on torch's current stream.  PyTorch supplies device memory
and streams.  The names and argument meanings follow ``include/pagedattn.h``.

The library is built in-tree by ``python -m paged_kv_cache_amd.build``; if it
is missing, importing the functions below raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; nothing in the environment redirects it.
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")
_lib = None

PA_DEVERR_BAD_PAGE = 1
PA_DEVERR_BAD_SLOT = 2
PA_DEVERR_BAD_POS = 4
PA_DEVERR_NO_FREE_PAGE = 8
PA_DEVERR_DUP_SLOT = 16
PA_DEVERR_REASSIGNED = 32
PA_DEVERR_STACK_FULL = 64
PA_DEVERR_BAD_PLAN = 128

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class PagedAttnError(RuntimeError):
    """A pagedattn call returned a negative status."""


def load():
    """Load libpagedattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [_I]
        lib.pa_page_bytes.restype = _I64
        lib.pa_page_bytes.argtypes = [_I, _I]
        lib.kv_scatter.restype = _I
        lib.kv_scatter.argtypes = [_P, _P, _I64, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _P, _P]
        lib.attn_prefill.restype = _I
        lib.attn_prefill.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _I,
                                     _F, _I, _P, _P, _P, _P]
        lib.attn_prefill_append.restype = _I
        lib.attn_prefill_append.argtypes = [_P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I,
                                            _I, _I, _F, _I, _P, _P, _P, _P]
        lib.attn_prefill_chunk.restype = _I
        lib.attn_prefill_chunk.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I,
                                           _I, _I, _F, _I, _P, _P, _P, _P]
        lib.attn_decode.restype = _I
        lib.attn_decode.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F,
                                    _I, _P, _SZ, _P, _P, _P, _P]
        lib.attn_decode_append.restype = _I
        lib.attn_decode_append.argtypes = [_P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I,
                                           _I, _F, _I, _P, _SZ, _P, _P, _P, _P]
        lib.attn_decode_noalloc.restype = _I
        lib.attn_decode_noalloc.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I,
                                            _F, _I, _P, _P, _P, _P]
        lib.attn_decode_workspace_size.restype = _SZ
        lib.attn_decode_workspace_size.argtypes = [_I, _I, _I, _I, _I]
        lib.attn_decode_whole_pages.restype = _I
        lib.attn_decode_whole_pages.argtypes = [_I, _I, _I, _I, _I]
        lib.kv_append.restype = _I
        lib.kv_append.argtypes = [_P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _I, _P, _I64, _P, _I, _I,
                                  _I, _I, _P, _I, _P, _I, _I, _P, _P]
        lib.kv_release.restype = _I
        lib.kv_release.argtypes = [_P, _I, _P, _I, _I, _I, _P, _I, _P, _P, _P]
        lib.attn_backward_dense.restype = _I
        lib.attn_backward_dense.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P,
                                            _P, _P, _SZ, _P]
        lib.attn_backward_workspace_size.restype = _SZ
        lib.attn_backward_workspace_size.argtypes = [_I, _I, _I]
        lib.attn_prefill_dense.restype = _I
        lib.attn_prefill_dense.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P]
        lib.attn_prefill_packed_plan.restype = _I
        lib.attn_prefill_packed_plan.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _I64, _P, _P, _P]
        lib.attn_prefill_packed.restype = _I
        lib.attn_prefill_packed.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _P, _I, _I64, _I, _I,
                                            _I, _F, _I, _P, _I64, _I64, _P, _SZ, _P, _P, _P, _P]
        lib.pa_clock_probe.restype = _I
        lib.pa_clock_probe.argtypes = [_P, _I, _I, _P]
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise PagedAttnError(f"{what}: {load().pa_status_string(rc).decode()} (status {rc})")


def _dev(t: torch.Tensor | None, dtype: torch.dtype | None = None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def page_bytes(n_kv_heads: int, head_dim: int) -> int:
    return int(load().pa_page_bytes(n_kv_heads, head_dim))


def clock_probe(n_waves: int = 4096, iters: int = 20000, stream=None) -> torch.Tensor:
    """Per-wave shader clock (GHz, float32 [n_waves]) while every SIMD issues bf16
    matrix products (a measurement aid, not part of the attention path)."""
    ghz = torch.zeros(n_waves, dtype=torch.float32, device=torch.device("cuda"))
    _check(load().pa_clock_probe(ghz.data_ptr(), n_waves, iters, _stream(stream)), "pa_clock_probe")
    return ghz


def _n_pages(kv_cache: torch.Tensor, n_kv_heads: int, head_dim: int) -> int:
    pb = page_bytes(n_kv_heads, head_dim)
    nbytes = kv_cache.numel() * kv_cache.element_size()
    if nbytes % pb:
        raise ValueError("kv_cache size is not a whole number of pages")
    return nbytes // pb


def kv_scatter(k: torch.Tensor, v: torch.Tensor, slot_ids: torch.Tensor, positions: torch.Tensor,
               kv_cache: torch.Tensor, block_table: torch.Tensor, layer: int,
               err: torch.Tensor | None = None, stream=None) -> None:
    """Write token rows k, v [N, Hkv, d] (bf16) into their pages of kv_cache."""
    N, Hkv, d = k.shape
    assert v.shape == k.shape and block_table.dim() == 3
    n_slots, n_layers, mbps = block_table.shape
    rc = load().kv_scatter(
        _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"), N,
        _dev(slot_ids, torch.int32, "slot_ids"), _dev(positions, torch.int32, "positions"),
        _dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, Hkv, d),
        _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer, Hkv, d,
        _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "kv_scatter")


def attn_prefill(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, layer: int,
                 seq_lens: torch.Tensor, n_kv_heads: int, scale: float, causal: bool = True,
                 slot_ids: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, err: torch.Tensor | None = None, stream=None,
                 q_lens: torch.Tensor | None = None):
    """Paged prefill of q [B, T, Hq, d]; returns (O [B, T, Hq, d] bf16, LSE [B, Hq, T] fp32).

    With q_lens, the queries of sequence b are the last q_lens[b] of its seq_lens[b] cached
    tokens (attn_prefill_chunk: prefix continuation, mixed prefill + decode batches)."""
    B, T, Hq, d = q.shape
    n_slots, n_layers, mbps = block_table.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    common = (_dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, n_kv_heads, d),
              _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer,
              _dev(slot_ids, torch.int32, "slot_ids"))
    tail = (B, T, Hq, n_kv_heads, d, float(scale), int(bool(causal)), _dev(out, torch.bfloat16, "out"),
            _dev(lse, torch.float32, "lse"), _dev(err, torch.int32, "err"), _stream(stream))
    if q_lens is None:
        rc = load().attn_prefill(_dev(q, torch.bfloat16, "q"), *common,
                                 _dev(seq_lens, torch.int32, "seq_lens"), *tail)
        _check(rc, "attn_prefill")
    else:
        rc = load().attn_prefill_chunk(_dev(q, torch.bfloat16, "q"), *common,
                                       _dev(q_lens, torch.int32, "q_lens"),
                                       _dev(seq_lens, torch.int32, "seq_lens"), *tail)
        _check(rc, "attn_prefill_chunk")
    return out, lse


class PackedPlan:
    """The work list of one packed batch (attn_prefill_packed_plan): ``host`` the
    int32 items, ``plan`` their device copy, the counts and the workspace bytes."""

    def __init__(self, host: np.ndarray, n_work: int, n_merge: int, workspace_bytes: int, device):
        self.host = host
        self.n_work = n_work
        self.n_merge = n_merge
        self.workspace_bytes = workspace_bytes
        self.plan = torch.from_numpy(host).to(device)

    def workspace(self) -> torch.Tensor | None:
        if self.workspace_bytes == 0:
            return None
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.plan.device)


def attn_prefill_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_cache: torch.Tensor,
                        block_table: torch.Tensor, layer: int, seq_lens: torch.Tensor, scale: float,
                        causal: bool = True, slot_ids: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        err: torch.Tensor | None = None, stream=None):
    """Prefill step in one launch: k, v [B, T, Hkv, d] (the prompts' K/V rows) are written to
    their pages and q [B, T, Hq, d] attends to them; returns (O [B, T, Hq, d] bf16,
    LSE [B, Hq, T] fp32), as kv_scatter of the prompt tokens followed by attn_prefill."""
    B, T, Hq, d = q.shape
    n_kv_heads = k.shape[2]
    if tuple(k.shape) != (B, T, n_kv_heads, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, T, Hkv, d] with q's B, T and d")
    n_slots, n_layers, mbps = block_table.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    rc = load().attn_prefill_append(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, n_kv_heads, d),
        _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer,
        _dev(slot_ids, torch.int32, "slot_ids"), _dev(seq_lens, torch.int32, "seq_lens"),
        B, T, Hq, n_kv_heads, d, float(scale), int(bool(causal)), _dev(out, torch.bfloat16, "out"),
        _dev(lse, torch.float32, "lse"), _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "attn_prefill_append")
    return out, lse


def prefill_packed_plan(q_lens, kv_lens, n_q_heads: int, n_kv_heads: int, head_dim: int,
                        causal: bool = True, device=None) -> PackedPlan:
    """Plan a packed batch on the host from host lengths (sequences, arrays of int)."""
    ql = np.ascontiguousarray(np.asarray(q_lens), dtype=np.int32)
    kv = np.ascontiguousarray(np.asarray(kv_lens), dtype=np.int32)
    if ql.shape != kv.shape or ql.ndim != 1:
        raise ValueError("q_lens and kv_lens must be 1-D and of one length")
    nw, nm, wb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    args = (ql.ctypes.data, kv.ctypes.data, ql.size, n_q_heads, n_kv_heads, head_dim, int(bool(causal)))
    lib = load()
    _check(lib.attn_prefill_packed_plan(*args, None, 0, ctypes.byref(nw), ctypes.byref(nm), ctypes.byref(wb)),
           "attn_prefill_packed_plan")
    host = np.zeros(max(6 * (nw.value + nm.value), 6), np.int32)
    _check(lib.attn_prefill_packed_plan(*args, host.ctypes.data, host.size, ctypes.byref(nw), ctypes.byref(nm),
                                        ctypes.byref(wb)), "attn_prefill_packed_plan")
    return PackedPlan(host, nw.value, nm.value, wb.value, device or torch.device("cuda"))


def attn_prefill_packed(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, layer: int,
                        kv_lens: torch.Tensor, q_start: torch.Tensor, plan: PackedPlan, n_kv_heads: int,
                        scale: float, causal: bool = True, slot_ids: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, err: torch.Tensor | None = None, stream=None):
    """Packed prefill of q [total_q, Hq, d] (sequence b's rows q_start[b] .. q_start[b+1]-1)
    by a plan from prefill_packed_plan; returns (O [total_q, Hq, d] bf16, LSE [total_q, Hq] fp32)."""
    total_q, Hq, d = q.shape
    B = kv_lens.numel()
    n_slots, n_layers, mbps = block_table.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(total_q, Hq, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = plan.workspace()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().attn_prefill_packed(
        _dev(q, torch.bfloat16, "q"), _dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, n_kv_heads, d),
        _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer,
        _dev(slot_ids, torch.int32, "slot_ids"), _dev(kv_lens, torch.int32, "kv_lens"),
        _dev(q_start, torch.int32, "q_start"), B, total_q, Hq, n_kv_heads, d, float(scale),
        int(bool(causal)), _dev(plan.plan, torch.int32, "plan"), plan.n_work, plan.n_merge,
        _dev(workspace, None, "workspace"), ws_bytes, _dev(out, torch.bfloat16, "out"),
        _dev(lse, torch.float32, "lse"), _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "attn_prefill_packed")
    return out, lse


def decode_workspace_size(B: int, Hq: int, Hkv: int, head_dim: int, max_ctx: int) -> int:
    return int(load().attn_decode_workspace_size(B, Hq, Hkv, head_dim, max_ctx))


def decode_whole_pages(B: int, Hq: int, Hkv: int, head_dim: int, max_ctx: int = 2048) -> bool:
    """Whether attn_decode (and attn_decode_noalloc) take the whole-page kernel
    for this shape on the current device (the library's own rule)."""
    return bool(load().attn_decode_whole_pages(B, Hq, Hkv, head_dim, max_ctx))


def decode_splits(B: int, Hq: int, Hkv: int, head_dim: int, max_ctx: int) -> int:
    """Workgroup splits per context of the per-head decode kernel for this
    shape (1: no workspace).  Read off the workspace size, whose fp32 partial
    outputs [B, Hq, splits, head_dim] dominate it.  Meaningless where
    decode_whole_pages() holds."""
    ws = decode_workspace_size(B, Hq, Hkv, head_dim, max_ctx)
    return 1 if ws == 0 else ws // (B * Hq * head_dim * 4)


def decode_workspace(B: int, Hq: int, Hkv: int, head_dim: int, max_ctx: int,
                     device=None) -> torch.Tensor:
    """A decode workspace of the size attn_decode needs for this shape (may be 16 B)."""
    n = max(decode_workspace_size(B, Hq, Hkv, head_dim, max_ctx), 16)
    return torch.empty(n, dtype=torch.uint8, device=device or torch.device("cuda"))


def attn_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, layer: int,
                ctx_lens: torch.Tensor, n_kv_heads: int, scale: float, max_ctx: int,
                slot_ids: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                err: torch.Tensor | None = None, stream=None):
    """Paged decode of q [B, Hq, d]; returns (O [B, Hq, d] bf16, LSE [B, Hq] fp32)."""
    B, Hq, d = q.shape
    n_slots, n_layers, mbps = block_table.shape
    if workspace is None:
        workspace = decode_workspace(B, Hq, n_kv_heads, d, max_ctx, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    rc = load().attn_decode(
        _dev(q, torch.bfloat16, "q"), _dev(kv_cache, None, "kv_cache"),
        _n_pages(kv_cache, n_kv_heads, d), _dev(block_table, torch.int32, "block_table"),
        n_slots, n_layers, mbps, layer, _dev(slot_ids, torch.int32, "slot_ids"),
        _dev(ctx_lens, torch.int32, "ctx_lens"), B, Hq, n_kv_heads, d, float(scale), int(max_ctx),
        _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _dev(out, torch.bfloat16, "out"), _dev(lse, torch.float32, "lse"),
        _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "attn_decode")
    return out, lse


def attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, kv_cache: torch.Tensor,
                       block_table: torch.Tensor, layer: int, ctx_lens: torch.Tensor, n_kv_heads: int,
                       scale: float, max_ctx: int, slot_ids: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, err: torch.Tensor | None = None, stream=None):
    """One decode step in one launch: k_new, v_new [B, Hkv, d] are written to the pages
    at position ctx_lens - 1 and attended to with the cached context; returns
    (O [B, Hq, d] bf16, LSE [B, Hq] fp32)."""
    B, Hq, d = q.shape
    n_slots, n_layers, mbps = block_table.shape
    if workspace is None:
        workspace = decode_workspace(B, Hq, n_kv_heads, d, max_ctx, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    rc = load().attn_decode_append(
        _dev(q, torch.bfloat16, "q"), _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
        _dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, n_kv_heads, d),
        _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer,
        _dev(slot_ids, torch.int32, "slot_ids"), _dev(ctx_lens, torch.int32, "ctx_lens"), B, Hq, n_kv_heads,
        d, float(scale), int(max_ctx), _dev(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _dev(out, torch.bfloat16, "out"),
        _dev(lse, torch.float32, "lse"), _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "attn_decode_append")
    return out, lse


def attn_decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                        layer: int, ctx_lens: torch.Tensor, n_kv_heads: int, scale: float,
                        max_ctx: int, out: torch.Tensor, lse: torch.Tensor,
                        slot_ids: torch.Tensor | None = None, err: torch.Tensor | None = None,
                        stream=None):
    """attn_decode without a workspace: the split partials go to the library's static
    device array.  out [B, Hq, d] bf16 and lse [B, Hq] fp32 are caller-provided (this
    wrapper allocates nothing either); returns (out, lse)."""
    B, Hq, d = q.shape
    n_slots, n_layers, mbps = block_table.shape
    rc = load().attn_decode_noalloc(
        _dev(q, torch.bfloat16, "q"), _dev(kv_cache, None, "kv_cache"),
        _n_pages(kv_cache, n_kv_heads, d), _dev(block_table, torch.int32, "block_table"),
        n_slots, n_layers, mbps, layer, _dev(slot_ids, torch.int32, "slot_ids"),
        _dev(ctx_lens, torch.int32, "ctx_lens"), B, Hq, n_kv_heads, d, float(scale), int(max_ctx),
        _dev(out, torch.bfloat16, "out"), _dev(lse, torch.float32, "lse"),
        _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "attn_decode_noalloc")
    return out, lse


def attn_prefill_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                       causal: bool = True, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, stream=None):
    """Unpaged prefill: q [B, T, Hq, d], k, v [B, T, Hkv, d]; returns (O, LSE [B, Hq, T])."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    rc = load().attn_prefill_dense(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        B, T, Hq, Hkv, d, float(scale), int(bool(causal)), _dev(out, torch.bfloat16, "out"),
        _dev(lse, torch.float32, "lse"), _stream(stream))
    _check(rc, "attn_prefill_dense")
    return out, lse


def kv_append(k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor, cos_t: torch.Tensor,
              sin_t: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, layer: int,
              free_pages: torch.Tensor, alloc_state: torch.Tensor,
              slot_ids: torch.Tensor | None = None, q: torch.Tensor | None = None,
              q_out: torch.Tensor | None = None, err: torch.Tensor | None = None,
              stream=None) -> torch.Tensor | None:
    """One decode step's cache writes: k, v [B, Hkv, d] (k before RoPE) for the token at
    positions[b]; pages popped from free_pages for opening tokens (block_table and
    alloc_state [2] int32 updated).  Rotates q [B, Hq, d] into q_out (default: a new
    tensor; pass q itself to rotate in place) and returns it (None without q)."""
    B, Hkv, d = k.shape
    assert v.shape == k.shape and block_table.dim() == 3 and cos_t.shape == sin_t.shape
    n_slots, n_layers, mbps = block_table.shape
    Hq = 0
    if q is not None:
        Hq = q.shape[1]
        if q_out is None:
            q_out = torch.empty_like(q)
    rc = load().kv_append(
        _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"), _dev(q, torch.bfloat16, "q"),
        _dev(q_out, torch.bfloat16, "q_out") if q is not None else None, Hq, B,
        _dev(slot_ids, torch.int32, "slot_ids"), _dev(positions, torch.int32, "positions"),
        _dev(cos_t, torch.float32, "cos_t"), _dev(sin_t, torch.float32, "sin_t"), cos_t.shape[0],
        _dev(kv_cache, None, "kv_cache"), _n_pages(kv_cache, Hkv, d),
        _dev(block_table, torch.int32, "block_table"), n_slots, n_layers, mbps, layer,
        _dev(free_pages, torch.int32, "free_pages"), free_pages.numel(),
        _dev(alloc_state, torch.int32, "alloc_state"), Hkv, d, _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "kv_append")
    return q_out if q is not None else None


def kv_release(slots: torch.Tensor, block_table: torch.Tensor, free_pages: torch.Tensor,
               alloc_state: torch.Tensor, err: torch.Tensor | None = None, stream=None) -> None:
    """Push the pages of the given slots back onto free_pages; their entries become -1."""
    n_slots, n_layers, mbps = block_table.shape
    rc = load().kv_release(
        _dev(slots, torch.int32, "slots"), slots.numel(), _dev(block_table, torch.int32, "block_table"),
        n_slots, n_layers, mbps, _dev(free_pages, torch.int32, "free_pages"), free_pages.numel(),
        _dev(alloc_state, torch.int32, "alloc_state"), _dev(err, torch.int32, "err"), _stream(stream))
    _check(rc, "kv_release")


def new_alloc_state(top: int, device=None) -> torch.Tensor:
    """The int32 [2] allocator state for kv_append / kv_release: {top, 0}."""
    return torch.tensor([int(top), 0], dtype=torch.int32, device=device or torch.device("cuda"))


def attn_backward_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                        dout: torch.Tensor, lse: torch.Tensor, scale: float, causal: bool = True,
                        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None):
    """Gradients of exact attention on contiguous q [B, T, Hq, d], k, v [B, T, Hkv, d], given
    the forward's o and lse [B, Hq, T] and the upstream gradient dout; returns (dq, dk, dv)."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        n = max(int(load().attn_backward_workspace_size(B, T, Hq)), 16)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    rc = load().attn_backward_dense(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(o, torch.bfloat16, "o"), _dev(dout, torch.bfloat16, "dout"), _dev(lse, torch.float32, "lse"),
        B, T, Hq, Hkv, d, float(scale), int(bool(causal)), _dev(dq, torch.bfloat16, "dq"),
        _dev(dk, torch.bfloat16, "dk"), _dev(dv, torch.bfloat16, "dv"), _dev(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "attn_backward_dense")
    return dq, dk, dv
