"""CPU oracle for paged causal GQA attention: test infrastructure only.

Only the test suite, the smoke check and the benchmark's ``cpu_baseline`` leg
may import this package.  The product path (``paged_kv_cache_amd``) never
does, and shares no code with it.

``oracle.c`` holds the arithmetic (fp64 plain definition of attention and the
page scatter); this module compiles it with gcc and marshals numpy arrays to
it.  Inputs are bf16 bit patterns (numpy uint16, or bf16 torch CPU tensors,
which are viewed, not rounded).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_D = ctypes.c_double


SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile oracle.c into liboracle.so (portable flags: the .so may run on another host).

    sanitize=True builds a host-only AddressSanitizer + UndefinedBehaviorSanitizer
    copy instead (``out``, default liboracle_san.so next to the source), which
    stops at the first error; a process that loads it needs libasan first in its
    library list (LD_PRELOAD), since the Python interpreter is not instrumented."""
    if sanitize:
        out = out or os.path.join(_HERE, "liboracle_san.so")
        subprocess.run(["gcc", "-std=c11", *SANITIZE_FLAGS, "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-Werror", _SRC, "-o", out, "-lm"], check=True)
        return out
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-Werror", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load(lib_path: str | None = None):
    """Load the compiled oracle (building it first if it is missing or stale)."""
    global _lib
    if lib_path is not None:
        return _bind(ctypes.CDLL(lib_path))
    if _lib is None:
        override = os.environ.get("ORACLE_LIB")      # a planted-mistake build (mutation tests)
        if override:
            _lib = _bind(ctypes.CDLL(override))
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    lib.oracle_num_threads.restype = _I
    lib.oracle_set_num_threads.argtypes = [_I]
    lib.oracle_page_bytes.restype = _I64
    lib.oracle_page_bytes.argtypes = [_I, _I]
    lib.oracle_kv_scatter.restype = _I64
    lib.oracle_kv_scatter.argtypes = [_P, _I64, _P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_attn_prefill.restype = _I64
    lib.oracle_attn_prefill.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _D, _I, _P, _I64, _P, _P]
    lib.oracle_attn_decode.restype = _I64
    lib.oracle_attn_decode.argtypes = [_P, _P, _I64, _P, _I, _I, _I, _I, _P, _P,
                                       _I, _I, _I, _I, _D, _P, _P]
    lib.oracle_round_bf16.restype = None
    lib.oracle_round_bf16.argtypes = [_P, _I64, _P]
    lib.oracle_rope.restype = _I64
    lib.oracle_rope.argtypes = [_P, _I64, _I, _I, _P, _P, _P, _I, _P]
    lib.oracle_kv_append.restype = _I
    lib.oracle_kv_append.argtypes = [_P, _I64, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _I,
                                     _P, _I, _I, _I, _I, _P, _P, _I, _I]
    lib.oracle_kv_release.restype = _I
    lib.oracle_kv_release.argtypes = [_P, _I, _P, _I, _I, _I, _P, _P, _I]
    lib.oracle_attn_dense_backward.restype = None
    lib.oracle_attn_dense_backward.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _D, _I, _P, _I,
                                               _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_attn_dense.restype = None
    lib.oracle_attn_dense.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _D, _I, _P, _I64, _P, _P]
    return lib


def _bits(x) -> np.ndarray:
    """uint16 bit patterns of a bf16 torch tensor or a uint16 numpy array (contiguous)."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    load().oracle_set_num_threads(int(n))


def page_bytes(n_kv_heads: int, head_dim: int) -> int:
    return int(load().oracle_page_bytes(n_kv_heads, head_dim))


def new_pool(n_pages: int, n_kv_heads: int, head_dim: int, fill: int) -> np.ndarray:
    """A host pool (uint8 bytes) whose every bf16 slot holds the bit pattern ``fill``."""
    words = n_pages * page_bytes(n_kv_heads, head_dim) // 2
    return np.full(words, fill, dtype=np.uint16).view(np.uint8)


def kv_scatter(pool: np.ndarray, n_pages: int, k, v, slot_ids, positions, block_table,
               layer: int, n_kv_heads: int, head_dim: int) -> int:
    """Write token K/V rows into ``pool`` in place; returns the count of skipped tokens."""
    kb, vb = _bits(k), _bits(v)
    n = kb.size // (n_kv_heads * head_dim)
    bt = _i32(block_table)
    assert bt.ndim == 3 and pool.dtype == np.uint8 and pool.flags.c_contiguous
    return int(load().oracle_kv_scatter(
        _ptr(pool), n_pages, _ptr(kb), _ptr(vb), n, _ptr(_i32(slot_ids)), _ptr(_i32(positions)),
        _ptr(bt), bt.shape[0], bt.shape[1], bt.shape[2], layer, n_kv_heads, head_dim))


def attn_prefill(q, pool: np.ndarray, n_pages: int, block_table, layer: int, slot_ids, seq_lens,
                 Hkv: int, scale: float, causal: bool, rows=None, q_lens=None):
    """Paged prefill rows (q_lens: queries are the last q_lens[b] of seq_lens[b] cached
    tokens; None: the whole sequence). Returns (O [n_rows,Hq,d] f64, LSE [n_rows,Hq] f64,
    bad_lookups)."""
    qb = _bits(q)
    B, T, Hq, d = q.shape
    bt = _i32(block_table)
    rws = None if rows is None else _i32(rows).reshape(-1, 2)
    n_rows = B * T if rws is None else rws.shape[0]
    O = np.empty((n_rows, Hq, d), np.float64)
    L = np.empty((n_rows, Hq), np.float64)
    bad = load().oracle_attn_prefill(
        _ptr(qb), _ptr(pool), n_pages, _ptr(bt), bt.shape[0], bt.shape[1], bt.shape[2], layer,
        _ptr(None if slot_ids is None else _i32(slot_ids)), _ptr(_i32(seq_lens)),
        _ptr(None if q_lens is None else _i32(q_lens)),
        B, T, Hq, Hkv, d, float(scale), int(bool(causal)), _ptr(rws), n_rows, _ptr(O), _ptr(L))
    return O, L, int(bad)


def attn_decode(q, pool: np.ndarray, n_pages: int, block_table, layer: int, slot_ids, ctx_lens,
                Hkv: int, scale: float):
    """Paged decode. Returns (O [B,Hq,d] f64, LSE [B,Hq] f64, bad_lookups)."""
    qb = _bits(q)
    B, Hq, d = q.shape
    bt = _i32(block_table)
    O = np.empty((B, Hq, d), np.float64)
    L = np.empty((B, Hq), np.float64)
    bad = load().oracle_attn_decode(
        _ptr(qb), _ptr(pool), n_pages, _ptr(bt), bt.shape[0], bt.shape[1], bt.shape[2], layer,
        _ptr(None if slot_ids is None else _i32(slot_ids)), _ptr(_i32(ctx_lens)),
        B, Hq, Hkv, d, float(scale), _ptr(O), _ptr(L))
    return O, L, int(bad)


def attn_dense(q, k, v, scale: float, causal: bool, rows=None):
    """Contiguous attention rows. Returns (O [n_rows,Hq,d] f64, LSE [n_rows,Hq] f64)."""
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    rws = None if rows is None else _i32(rows).reshape(-1, 2)
    n_rows = B * T if rws is None else rws.shape[0]
    O = np.empty((n_rows, Hq, d), np.float64)
    L = np.empty((n_rows, Hq), np.float64)
    load().oracle_attn_dense(_ptr(qb), _ptr(kb), _ptr(vb), B, T, Hq, Hkv, d, float(scale),
                             int(bool(causal)), _ptr(rws), n_rows, _ptr(O), _ptr(L))
    return O, L


def attn_dense_backward(q, k, v, dout, scale: float, causal: bool, with_abs: bool = False,
                        pairs=None):
    """Gradients of sum(O * dout) w.r.t. q, k, v (contiguous [B,T,H,d] bf16 inputs).

    Returns (dQ, dK, dV) in float64; with with_abs also (aQ, aK, aV) -- the same sums
    over the absolute values of their terms -- and (eQ, eK), the bounds on how far dQ,
    dK move when D is computed from a bf16-rounded forward output.  pairs: evaluate only
    these (b, kv head) pairs (the other outputs are 0)."""
    qb, kb, vb, ob = _bits(q), _bits(k), _bits(v), _bits(dout)
    B, T, Hq, d = qb.shape
    Hkv = kb.shape[2]
    dQ = np.empty((B, T, Hq, d), np.float64)
    dK = np.empty((B, T, Hkv, d), np.float64)
    dV = np.empty((B, T, Hkv, d), np.float64)
    a = [np.empty_like(x) for x in (dQ, dK, dV, dQ, dK)] if with_abs else [None] * 5
    pr = None if pairs is None else _i32(pairs).reshape(-1, 2)
    load().oracle_attn_dense_backward(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(ob), B, T, Hq, Hkv, d,
                                      float(scale), int(bool(causal)), _ptr(pr),
                                      0 if pr is None else pr.shape[0], _ptr(dQ), _ptr(dK), _ptr(dV),
                                      _ptr(a[0]), _ptr(a[1]), _ptr(a[2]), _ptr(a[3]), _ptr(a[4]))
    return (dQ, dK, dV, *a) if with_abs else (dQ, dK, dV)


# Error bits of the device flag (the library's ABI values).
ERR_BAD_PAGE, ERR_BAD_SLOT, ERR_BAD_POS = 1, 2, 4
ERR_NO_FREE_PAGE, ERR_DUP_SLOT, ERR_REASSIGNED, ERR_STACK_FULL = 8, 16, 32, 64


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of each float64 value, as uint16 bit patterns."""
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(xa.shape, np.uint16)
    load().oracle_round_bf16(_ptr(xa), xa.size, _ptr(out))
    return out


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def rope(x, positions, cos_t, sin_t) -> np.ndarray:
    """RoPE of x [n_tok, n_heads, d] (bf16 bits) at positions: float64, unrounded."""
    xb = _bits(x)
    n_tok, n_heads, d = xb.shape
    ct, st = _f32(cos_t), _f32(sin_t)
    assert ct.shape == st.shape and ct.shape[1] == d // 2
    out = np.empty((n_tok, n_heads, d), np.float64)
    load().oracle_rope(_ptr(xb), n_tok, n_heads, d, _ptr(_i32(positions)), _ptr(ct), _ptr(st),
                       ct.shape[0], _ptr(out))
    return out


def kv_append(pool: np.ndarray, n_pages: int, k, v, positions, cos_t, sin_t, block_table: np.ndarray,
              layer: int, free_pages, top: int, slot_ids=None, q=None):
    """One decode step's writes (pool and block_table updated in place).

    Returns (q_out bits or None, new top, error bits)."""
    kb, vb = _bits(k), _bits(v)
    B, Hkv, d = kb.shape
    assert block_table.dtype == np.int32 and block_table.flags.c_contiguous and block_table.ndim == 3
    ct, st = _f32(cos_t), _f32(sin_t)
    qb = None if q is None else _bits(q)
    Hq = 0 if qb is None else qb.shape[1]
    q_out = None if qb is None else qb.copy()
    fp = _i32(free_pages)
    t = np.array([top], np.int32)
    errs = load().oracle_kv_append(
        _ptr(pool), n_pages, _ptr(kb), _ptr(vb), _ptr(qb), _ptr(q_out), Hq, B,
        _ptr(None if slot_ids is None else _i32(slot_ids)), _ptr(_i32(positions)), _ptr(ct), _ptr(st),
        ct.shape[0], _ptr(block_table), block_table.shape[0], block_table.shape[1], block_table.shape[2],
        layer, _ptr(fp), _ptr(t), Hkv, d)
    return q_out, int(t[0]), int(errs)


def kv_release(slots, block_table: np.ndarray, free_pages: np.ndarray, top: int):
    """Push the pages of finished slots back onto the free stack (both updated in place).

    Returns (new top, error bits)."""
    assert block_table.dtype == np.int32 and block_table.flags.c_contiguous and block_table.ndim == 3
    assert free_pages.dtype == np.int32 and free_pages.flags.c_contiguous
    sl = _i32(slots)
    t = np.array([top], np.int32)
    errs = load().oracle_kv_release(_ptr(sl), sl.size, _ptr(block_table), block_table.shape[0],
                                    block_table.shape[1], block_table.shape[2], _ptr(free_pages),
                                    _ptr(t), free_pages.size)
    return int(t[0]), int(errs)


# Convenience wrappers over the seeded cases (duck-typed: any object with the
# same attribute names works).

def pool_for(case) -> np.ndarray:
    c = case.cache
    return new_pool(c.n_pages, c.n_kv_heads, c.head_dim, c.page_fill)


def scatter_tokens(pool: np.ndarray, cache, tokens) -> int:
    return kv_scatter(pool, cache.n_pages, tokens.k, tokens.v, tokens.slot_ids, tokens.positions,
                      cache.block_table, cache.layer, cache.n_kv_heads, cache.head_dim)


def prefill_case(case, rows=None, pool: np.ndarray | None = None):
    """Scatter the prompt into a fresh pool, then evaluate prefill rows; returns (O, LSE, pool)."""
    if pool is None:
        pool = pool_for(case)
        bad = scatter_tokens(pool, case.cache, case.tokens)
        assert bad == 0
    c = case.cache
    O, L, bad = attn_prefill(case.q, pool, c.n_pages, c.block_table, c.layer, case.slot_ids,
                             case.seq_lens, c.n_kv_heads, case.scale, case.causal, rows,
                             q_lens=getattr(case, "q_lens", None))
    assert bad == 0
    return O, L, pool


def decode_case(case, pool: np.ndarray | None = None):
    """Scatter context and newest tokens into a fresh pool, then decode; returns (O, LSE, pool)."""
    if pool is None:
        pool = pool_for(case)
        assert scatter_tokens(pool, case.cache, case.context) == 0
        assert scatter_tokens(pool, case.cache, case.new_tokens) == 0
    c = case.cache
    O, L, bad = attn_decode(case.q, pool, c.n_pages, c.block_table, c.layer, case.slot_ids,
                            case.ctx_lens, c.n_kv_heads, case.scale)
    assert bad == 0
    return O, L, pool


def dense_case(case, rows=None):
    return attn_dense(case.q, case.k, case.v, case.scale, case.causal, rows)
