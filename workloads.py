"""Seeded synthetic inputs for the paged causal GQA attention path.

This module is shared by the tests, by ``bench.py`` and by the smoke check.
It holds no attention arithmetic: it only draws random tensors and lengths
and does the caller-side bookkeeping a serving loop would do (hand physical
pages to (slot, layer, logical block) entries of a block table).

Conventions (the pages fix none of them, so the plainest reading is used):

* Tensors come from one CPU ``torch.Generator().manual_seed(seed)``; ``randn``
  is drawn in fp32 in the order Q, K, V and rounded to bfloat16
  (round-to-nearest-even, torch's ``.to(torch.bfloat16)``).
* Physical pages come from ``numpy.random.default_rng(seed).permutation(n_pages)``
  taken in order; decode context lengths come from the same numpy generator
  (``integers(1, max_ctx + 1)``) after the permutation.
* A block-table entry of -1 means "no page assigned" (tiny-vllm part 6,
  "block table" section).
* The initial pool content is a fill pattern (``page_fill``, a bf16 bit
  pattern): by default a quiet NaN, so any read of a byte that was never
  written poisons the result.

Page geometry used for sizing the pool (tiny-vllm part 6, "Block contents"
section): 16 tokens per page, K then V, each ``16 * n_kv_heads * head_dim``
bf16 values, so a page holds ``2 * 16 * n_kv_heads * head_dim * 2`` bytes
(32768 B at 8 KV heads x 64).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_TOKENS = 16
BF16_QNAN = 0x7FC0          # quiet NaN bit pattern for the pool fill
BF16_ZERO = 0x0000


def page_bytes(n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one physical page (K block then V block) for sizing buffers."""
    return 2 * PAGE_TOKENS * n_kv_heads * head_dim * 2


def _randn_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw uint16 bit patterns of a bf16 CPU tensor (a view, no rounding)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class PagedCache:
    """Caller-side description of a paged KV pool and its block table."""

    n_pages: int
    n_kv_heads: int
    head_dim: int
    block_table: np.ndarray          # int32 [n_slots, n_layers, max_blocks_per_seq]
    layer: int
    page_fill: int = BF16_QNAN

    @property
    def n_slots(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def n_layers(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[2])

    @property
    def page_bytes(self) -> int:
        return page_bytes(self.n_kv_heads, self.head_dim)

    @property
    def pool_bytes(self) -> int:
        return self.n_pages * self.page_bytes


@dataclass
class TokenBatch:
    """K/V rows of a set of tokens and where they belong (slot, position)."""

    k: torch.Tensor                  # [N, Hkv, d] bf16
    v: torch.Tensor                  # [N, Hkv, d] bf16
    slot_ids: np.ndarray             # int32 [N]
    positions: np.ndarray            # int32 [N]


@dataclass
class PrefillCase:
    name: str
    q: torch.Tensor                  # [B, T, Hq, d] bf16
    tokens: TokenBatch               # every prompt token, (b, t) order
    seq_lens: np.ndarray             # int32 [B]
    slot_ids: np.ndarray             # int32 [B]: batch row -> block-table slot
    cache: PagedCache
    scale: float
    causal: bool = True
    # queries are the last q_lens[b] of the seq_lens[b] cached tokens (None: all of them)
    q_lens: np.ndarray | None = None

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def T(self) -> int:
        return int(self.q.shape[1])

    @property
    def Hq(self) -> int:
        return int(self.q.shape[2])

    @property
    def d(self) -> int:
        return int(self.q.shape[3])


@dataclass
class DecodeCase:
    name: str
    q: torch.Tensor                  # [B, Hq, d] bf16: query of the newest token
    context: TokenBatch              # all tokens already in the cache (positions < ctx-1)
    new_tokens: TokenBatch           # the newest token of each sequence (position ctx-1)
    ctx_lens: np.ndarray             # int32 [B], includes the newest token
    slot_ids: np.ndarray             # int32 [B]
    cache: PagedCache
    scale: float

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def Hq(self) -> int:
        return int(self.q.shape[1])

    @property
    def d(self) -> int:
        return int(self.q.shape[2])

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max()) if len(self.ctx_lens) else 0


@dataclass
class DenseCase:
    name: str
    q: torch.Tensor                  # [B, T, Hq, d]
    k: torch.Tensor                  # [B, T, Hkv, d]
    v: torch.Tensor
    scale: float
    causal: bool
    dout: torch.Tensor | None = None  # [B, T, Hq, d]: upstream gradient (backward cases)


def _assign_pages(perm: np.ndarray, cursor: int, n_blocks: int) -> tuple[np.ndarray, int]:
    pages = perm[cursor:cursor + n_blocks]
    if len(pages) != n_blocks:
        raise ValueError("page pool too small for the requested contexts")
    return pages.astype(np.int32), cursor + n_blocks


def _empty_table(n_slots: int, n_layers: int, mbps: int) -> np.ndarray:
    return np.full((n_slots, n_layers, mbps), -1, dtype=np.int32)


def make_prefill(name: str, *, B: int, T: int, Hq: int, Hkv: int, d: int,
                 n_pages: int, seed: int = 0, seq_lens=None, scale: float | None = None,
                 causal: bool = True, n_layers: int = 1, layer: int = 0,
                 mbps: int | None = None, n_slots: int | None = None,
                 slot_ids=None, page_fill: int = BF16_QNAN,
                 fill_other_layers: bool = False) -> PrefillCase:
    """Prompt of B sequences (padded length T) with K/V to be scattered into pages.

    Every sequence's logical blocks get consecutive entries of one random page
    permutation.  With ``fill_other_layers`` the unused layers of the table
    also get pages (so a wrong layer stride reads the wrong, NaN-poisoned pages).
    """
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = _randn_bf16(gen, (B, T, Hq, d))
    k = _randn_bf16(gen, (B, T, Hkv, d))
    v = _randn_bf16(gen, (B, T, Hkv, d))
    perm = rng.permutation(n_pages)
    if seq_lens is None:
        seq_lens = np.full(B, T, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,) and int(seq_lens.max(initial=0)) <= T
    mbps = mbps if mbps is not None else -(-T // PAGE_TOKENS)
    n_slots = n_slots if n_slots is not None else B
    slot_ids = np.arange(B, dtype=np.int32) if slot_ids is None else np.asarray(slot_ids, np.int32)
    table = _empty_table(n_slots, n_layers, mbps)
    cursor = 0
    for b in range(B):
        nb = -(-int(seq_lens[b]) // PAGE_TOKENS)
        pages, cursor = _assign_pages(perm, cursor, nb)
        table[slot_ids[b], layer, :nb] = pages
    if fill_other_layers:
        for b in range(B):
            for lyr in range(n_layers):
                if lyr == layer:
                    continue
                nb = -(-int(seq_lens[b]) // PAGE_TOKENS)
                pages, cursor = _assign_pages(perm, cursor, nb)
                table[slot_ids[b], lyr, :nb] = pages
    bs, ts = [], []
    for b in range(B):
        bs.append(np.full(int(seq_lens[b]), b))
        ts.append(np.arange(int(seq_lens[b])))
    bi = np.concatenate(bs) if bs else np.zeros(0, np.int64)
    ti = np.concatenate(ts) if ts else np.zeros(0, np.int64)
    tokens = TokenBatch(k=k[bi, ti].contiguous(), v=v[bi, ti].contiguous(),
                        slot_ids=slot_ids[bi].astype(np.int32), positions=ti.astype(np.int32))
    cache = PagedCache(n_pages=n_pages, n_kv_heads=Hkv, head_dim=d, block_table=table,
                       layer=layer, page_fill=page_fill)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(np.float32(scale))
    return PrefillCase(name=name, q=q, tokens=tokens, seq_lens=seq_lens, slot_ids=slot_ids,
                       cache=cache, scale=scale, causal=causal)


def make_chunk(name: str, *, B: int, Hq: int, Hkv: int, d: int, n_pages: int, kv_lens, q_lens,
               seed: int = 0, scale: float | None = None, causal: bool = True, n_layers: int = 1,
               layer: int = 0, mbps: int | None = None, n_slots: int | None = None, slot_ids=None,
               page_fill: int = BF16_QNAN) -> PrefillCase:
    """A prompt chunk continuing a cached prefix: sequence b has kv_lens[b] tokens in the
    cache (``tokens`` holds all of them, prefix and chunk), and its queries are the last
    q_lens[b] of them, padded to T = max(q_lens).  The draws are those of ``make_prefill``
    with T = max(kv_lens): query row t of the chunk is the full prompt's row
    kv_lens[b] - q_lens[b] + t."""
    kv_lens = np.asarray(kv_lens, np.int32)
    q_lens = np.asarray(q_lens, np.int32)
    assert kv_lens.shape == (B,) and q_lens.shape == (B,) and np.all(q_lens <= kv_lens)
    full = make_prefill(name, B=B, T=max(int(kv_lens.max(initial=0)), 1), Hq=Hq, Hkv=Hkv, d=d,
                        n_pages=n_pages, seed=seed, seq_lens=kv_lens, scale=scale, causal=causal,
                        n_layers=n_layers, layer=layer, mbps=mbps, n_slots=n_slots,
                        slot_ids=slot_ids, page_fill=page_fill)
    T = max(int(q_lens.max(initial=0)), 1)
    q = torch.zeros(B, T, Hq, d, dtype=torch.bfloat16)
    for b in range(B):
        ql, kv = int(q_lens[b]), int(kv_lens[b])
        q[b, :ql] = full.q[b, kv - ql:kv]
    full.q = q
    full.q_lens = q_lens
    return full


def llama_chunk(seed: int = 0) -> PrefillCase:
    """Prefix continuation: 2 sequences with 2048 cached tokens each take a 2048-token
    chunk (4096 in the cache after it), 32/8/64, 2 GiB pool."""
    return make_chunk("chunk_llama_b2_prefix2048_q2048", B=2, Hq=LLAMA_HQ, Hkv=LLAMA_HKV, d=LLAMA_D,
                      n_pages=POOL_PAGES, kv_lens=[4096, 4096], q_lens=[2048, 2048], seed=seed,
                      scale=1.0 / 8.0, mbps=256)


def mixed_batch(seed: int = 0) -> PrefillCase:
    """Mixed prefill + decode in one call: 2 prompt chunks of 512 tokens (after 1000 and
    3000 cached tokens) and 62 decode rows (one query each, contexts U[1, 2048])."""
    rng = np.random.default_rng(seed + 31)
    dec = rng.integers(1, 2049, size=62)
    kv = np.concatenate([[1512, 3512], dec]).astype(np.int32)
    ql = np.concatenate([[512, 512], np.ones(62, np.int64)]).astype(np.int32)
    return make_chunk("mixed_b64_2chunks512_62decode", B=64, Hq=LLAMA_HQ, Hkv=LLAMA_HKV, d=LLAMA_D,
                      n_pages=POOL_PAGES, kv_lens=kv, q_lens=ql, seed=seed, scale=1.0 / 8.0, mbps=256)


def make_decode(name: str, *, B: int, Hq: int, Hkv: int, d: int, n_pages: int,
                ctx_lens=None, max_ctx: int = 2048, seed: int = 0,
                scale: float | None = None, n_layers: int = 1, layer: int = 0,
                mbps: int | None = None, n_slots: int | None = None, slot_ids=None,
                page_fill: int = BF16_QNAN) -> DecodeCase:
    """One decode step: B sequences whose caches hold ctx_lens[b] tokens each.

    ``context`` holds positions 0..ctx-2 (already cached), ``new_tokens`` the
    token at position ctx-1 that the step appends before attending.
    """
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)
    if ctx_lens is None:
        ctx_lens = rng.integers(1, max_ctx + 1, size=B)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    assert ctx_lens.shape == (B,)
    n_tok = int(ctx_lens.sum())
    q = _randn_bf16(gen, (B, Hq, d))
    k = _randn_bf16(gen, (n_tok, Hkv, d))
    v = _randn_bf16(gen, (n_tok, Hkv, d))
    mbps = mbps if mbps is not None else max(1, -(-int(ctx_lens.max(initial=1)) // PAGE_TOKENS))
    n_slots = n_slots if n_slots is not None else B
    slot_ids = np.arange(B, dtype=np.int32) if slot_ids is None else np.asarray(slot_ids, np.int32)
    table = _empty_table(n_slots, n_layers, mbps)
    cursor = 0
    tok_slot = np.empty(n_tok, np.int32)
    tok_pos = np.empty(n_tok, np.int32)
    is_new = np.zeros(n_tok, bool)
    off = 0
    for b in range(B):
        c = int(ctx_lens[b])
        nb = -(-c // PAGE_TOKENS)
        pages, cursor = _assign_pages(perm, cursor, nb)
        table[slot_ids[b], layer, :nb] = pages
        tok_slot[off:off + c] = slot_ids[b]
        tok_pos[off:off + c] = np.arange(c)
        if c:
            is_new[off + c - 1] = True
        off += c
    old = ~is_new
    context = TokenBatch(k=k[torch.from_numpy(old)].contiguous(), v=v[torch.from_numpy(old)].contiguous(),
                         slot_ids=tok_slot[old], positions=tok_pos[old])
    new = TokenBatch(k=k[torch.from_numpy(is_new)].contiguous(), v=v[torch.from_numpy(is_new)].contiguous(),
                     slot_ids=tok_slot[is_new], positions=tok_pos[is_new])
    cache = PagedCache(n_pages=n_pages, n_kv_heads=Hkv, head_dim=d, block_table=table,
                       layer=layer, page_fill=page_fill)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(np.float32(scale))
    return DecodeCase(name=name, q=q, context=context, new_tokens=new, ctx_lens=ctx_lens,
                      slot_ids=slot_ids, cache=cache, scale=scale)


def make_dense(name: str, *, B: int, T: int, Hq: int, Hkv: int, d: int, causal: bool,
               seed: int = 0, scale: float | None = None, grad: bool = False) -> DenseCase:
    """Contiguous Q, K, V [B, T, H, d]; with ``grad`` also the upstream gradient dO
    (drawn after V from the same generator, so Q, K, V are those of the forward case)."""
    gen = torch.Generator().manual_seed(seed)
    q = _randn_bf16(gen, (B, T, Hq, d))
    k = _randn_bf16(gen, (B, T, Hkv, d))
    v = _randn_bf16(gen, (B, T, Hkv, d))
    dout = _randn_bf16(gen, (B, T, Hq, d)) if grad else None
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else float(np.float32(scale))
    return DenseCase(name=name, q=q, k=k, v=v, scale=scale, causal=causal, dout=dout)


# ---------------------------------------------------------------------------
# The named workloads (Llama-3.2-1B attention shape: 32 q heads, 8 KV heads,
# head_dim 64; pool of 65536 pages of 32768 B = 2 GiB).
# ---------------------------------------------------------------------------

LLAMA_HQ, LLAMA_HKV, LLAMA_D = 32, 8, 64
POOL_PAGES = 65536


def tiny_prefill(seed: int = 0) -> PrefillCase:
    """17-token single-sequence prompt, one layer, 2 random pages of a 64-page pool."""
    return make_prefill("prefill_17tok", B=1, T=17, Hq=LLAMA_HQ, Hkv=LLAMA_HKV, d=LLAMA_D,
                        n_pages=64, seed=seed, scale=1.0 / 8.0, mbps=128)


def llama_prefill(seed: int = 0) -> PrefillCase:
    """Causal prefill, batch 2 x 2048 tokens, 32/8/64, 2 GiB pool, 128 blocks each."""
    return make_prefill("prefill_llama_b2_t2048", B=2, T=2048, Hq=LLAMA_HQ, Hkv=LLAMA_HKV,
                        d=LLAMA_D, n_pages=POOL_PAGES, seed=seed, scale=1.0 / 8.0, mbps=128)


def llama_decode(seed: int = 0) -> DecodeCase:
    """Decode step, 64 sequences with context uniform in [1, 2048], 2 GiB pool."""
    return make_decode("decode_llama_b64_ctx_u1_2048", B=64, Hq=LLAMA_HQ, Hkv=LLAMA_HKV,
                       d=LLAMA_D, n_pages=POOL_PAGES, max_ctx=2048, seed=seed,
                       scale=1.0 / 8.0, mbps=128)


def long_decode(seed: int = 0) -> DecodeCase:
    """Long-context decode: 4 sequences of 16384 tokens (1024 pages each)."""
    return make_decode("decode_long_b4_ctx16384", B=4, Hq=LLAMA_HQ, Hkv=LLAMA_HKV, d=LLAMA_D,
                       n_pages=POOL_PAGES, ctx_lens=[16384] * 4, seed=seed, scale=1.0 / 8.0,
                       mbps=1024)


def long_prefill(seed: int = 0) -> DenseCase:
    """Low-occupancy long prefill: batch 1, 16384 tokens, 16 heads x 128, causal."""
    return make_dense("dense_long_b1_t16384_h16_d128_causal", B=1, T=16384, Hq=16, Hkv=16,
                      d=128, causal=True, seed=seed)


FA2_SEQLENS = (512, 1024, 2048, 4096, 8192, 16384)
FA2_HEADS = ((64, 32), (128, 16))      # (head_dim, heads): hidden 2048


def fa2_dense(T: int, d: int, causal: bool, seed: int = 0, grad: bool = False) -> DenseCase:
    """FlashAttention-2 benchmark shape: hidden 2048, batch x seqlen = 16384 tokens, MHA
    (with ``grad``: plus the upstream gradient, for the backward)."""
    H = 2048 // d
    return make_dense(f"dense_fa2_t{T}_d{d}_{'causal' if causal else 'full'}", B=16384 // T, T=T,
                      Hq=H, Hkv=H, d=d, causal=causal, seed=seed, grad=grad)


# ---------------------------------------------------------------------------
# Decode append: RoPE angle tables and a cache state ready for one more token.
# ---------------------------------------------------------------------------

def rope_tables(max_pos: int, d: int, base: float = 500000.0) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [max_pos, d/2] fp32 of the angles pos * base^(-2i/d).

    The pages build such tables once at start-up and only look them up; they
    do not print the frequencies, so the usual geometric progression is used
    here with Llama 3's base.  Any table is a valid input.
    """
    i = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def random_angle_tables(max_pos: int, d: int, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [max_pos, d/2] fp32 of angles drawn uniformly in [-pi, pi)."""
    rng = np.random.default_rng(seed + 7919)
    ang = rng.uniform(-np.pi, np.pi, size=(max_pos, d // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclass
class AppendCase:
    """A cache whose sequences hold ctx_lens[b] - 1 tokens, plus the next token of each.

    ``block_table`` has pages for the cached tokens only: the block a new token
    opens (position % 16 == 0) is still -1.  ``free_pages`` is the stack of
    every page not in the table (a permutation tail), all of it free (top =
    its length); pops take from the back.
    """

    name: str
    decode: DecodeCase               # q (before RoPE), context, new tokens (K before RoPE)
    block_table: np.ndarray          # int32 table before the append
    free_pages: np.ndarray           # int32 [n_free]
    cos_t: np.ndarray                # fp32 [max_pos, d/2]
    sin_t: np.ndarray

    @property
    def top(self) -> int:
        return int(self.free_pages.shape[0])


def make_append(name: str, *, B: int, Hq: int, Hkv: int, d: int, n_pages: int, ctx_lens=None,
                max_ctx: int = 2048, seed: int = 0, mbps: int | None = None, n_layers: int = 1,
                layer: int = 0, n_slots: int | None = None, slot_ids=None,
                random_angles: bool = False, page_fill: int = BF16_QNAN) -> AppendCase:
    dc = make_decode(name, B=B, Hq=Hq, Hkv=Hkv, d=d, n_pages=n_pages, ctx_lens=ctx_lens,
                     max_ctx=max_ctx, seed=seed, n_layers=n_layers, layer=layer, mbps=mbps,
                     n_slots=n_slots, slot_ids=slot_ids, page_fill=page_fill)
    table = dc.cache.block_table.copy()
    for b in range(B):
        p = int(dc.ctx_lens[b]) - 1
        if p >= 0 and p % PAGE_TOKENS == 0:
            table[dc.slot_ids[b], layer, p // PAGE_TOKENS] = -1
    used = set(int(x) for x in table.ravel() if x >= 0)
    rng = np.random.default_rng(seed + 104729)
    free = np.array([p for p in rng.permutation(n_pages) if int(p) not in used], dtype=np.int32)
    max_pos = int(table.shape[2]) * PAGE_TOKENS
    if random_angles:
        cos_t, sin_t = random_angle_tables(max_pos, d, seed)
    else:
        cos_t, sin_t = rope_tables(max_pos, d)
    return AppendCase(name=name, decode=dc, block_table=table, free_pages=free, cos_t=cos_t,
                      sin_t=sin_t)


def llama_append(seed: int = 0) -> AppendCase:
    """Decode append for the 64-sequence Llama decode batch (context U[1, 2048])."""
    return make_append("append_llama_b64", B=64, Hq=LLAMA_HQ, Hkv=LLAMA_HKV, d=LLAMA_D,
                       n_pages=POOL_PAGES, max_ctx=2048, seed=seed, mbps=128)
