"""The C-ABI library loads and exports what include/pagedattn.h declares; host
argument checks reject bad calls before anything is launched (CPU only)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", src, re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ["kv_scatter", "attn_prefill", "attn_decode", "attn_prefill_dense",
              "attn_decode_workspace_size", "attn_decode_whole_pages", "pa_status_string", "pa_page_bytes", "kv_append",
              "kv_release", "attn_prefill_chunk", "attn_backward_dense",
              "attn_backward_workspace_size"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pa.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in pagedattn.h but not exported"


def test_page_bytes_and_status_strings():
    assert pa.page_bytes(8, 64) == 32768
    assert pa.page_bytes(2, 128) == 2 * 16 * 2 * 128 * 2
    lib = pa.load()
    for s in range(0, -9, -1):
        assert lib.pa_status_string(s).decode() not in ("", "unknown status")
    assert lib.pa_status_string(5).decode() == "unknown status"


def test_decode_workspace_size():
    # head_dim 128 (per-head kernel): a batch that fills the GPU needs no
    # cross-workgroup partials; a few long contexts are split across
    # workgroups (O and LSE partials)
    assert pa.decode_workspace_size(64, 32, 8, 128, 2048) == 0
    assert pa.decode_workspace_size(4, 32, 8, 128, 16384) >= 4 * 32 * 2 * (128 + 1) * 4
    assert pa.decode_workspace_size(0, 32, 8, 64, 2048) == 0
    assert pa.decode_splits(64, 32, 8, 128, 2048) == 1
    assert pa.decode_splits(4, 32, 8, 128, 16384) >= 2


def test_decode_whole_page_workspace():
    # 8 kv heads of head_dim 64 (group <= 8, B <= 512): one workgroup per CU
    # (256 here, also the count assumed without a device), a partial per
    # (sequence, workgroup) in slot b + g < 256 + B, plus [B][2] slot ranges
    for B, Hq, max_ctx in ((4, 32, 16384), (32, 32, 2048), (128, 32, 2048), (512, 32, 2048), (3, 8, 100)):
        assert pa.decode_whole_pages(B, Hq, 8, 64, max_ctx)
        n_wg = min(256, B * ((max_ctx + 15) // 16))
        assert pa.decode_workspace_size(B, Hq, 8, 64, max_ctx) >= (n_wg + B) * Hq * (64 + 1) * 4 + B * 8
    # a short batch uses fewer workgroups than CUs: 3 sequences of up to 100
    # tokens have at most 21 pages
    assert pa.decode_workspace_size(3, 8, 8, 64, 100) < (256 + 3) * 8 * 65 * 4
    # one to two (sequence, kv head) units per CU: the per-head kernel
    assert not pa.decode_whole_pages(33, 32, 8, 64)
    assert not pa.decode_whole_pages(64, 32, 8, 64)
    assert pa.decode_whole_pages(65, 32, 8, 64)
    assert not pa.decode_whole_pages(513, 32, 8, 64)       # the length scan holds 512
    assert not pa.decode_whole_pages(16, 128, 8, 64)       # group 16
    assert not pa.decode_whole_pages(16, 32, 8, 128)
    assert not pa.decode_whole_pages(16, 16, 4, 64)
    assert not pa.decode_whole_pages(0, 32, 8, 64)
    # a workgroup resolves at most 1024 pages of its range up front: batches
    # of more than 1024 pages per CU take the per-head kernel
    assert pa.decode_whole_pages(512, 32, 8, 64, 512 * 16)
    assert not pa.decode_whole_pages(512, 32, 8, 64, 512 * 16 + 16)


def test_decode_split_policy_one_workgroup_per_cu():
    # per-head kernel (here head_dim 128): splits give every CU (256 on this
    # part, also the count assumed without a device) one workgroup: B * Hkv *
    # splits = 256, never below 2 chunks of 32 tokens per wavefront (512 tokens
    # per split)
    assert pa.decode_splits(4, 32, 8, 128, 16384) == 8      # 32 groups x 8
    assert pa.decode_splits(16, 32, 8, 128, 2048) == 2      # 128 groups x 2
    assert pa.decode_splits(1, 32, 8, 128, 3000) == 6       # 32 wanted, 3000 / 512 allowed
    assert pa.decode_splits(1, 32, 8, 128, 100) == 1
    assert pa.decode_splits(32, 32, 8, 128, 2048) == 1      # 256 groups already


P = ctypes.c_void_p


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def test_host_checks_reject_bad_arguments():
    lib = pa.load()
    good = _fake()
    # NULL cache
    assert lib.kv_scatter(good, good, 1, good, good, None, 64, good, 1, 1, 128, 0, 8, 64, None, None) == -1
    # layer out of range
    assert lib.kv_scatter(good, good, 1, good, good, good, 64, good, 1, 1, 128, 1, 8, 64, None, None) == -2
    # misaligned k
    assert lib.kv_scatter(_fake(0x10002), good, 1, good, good, good, 64, good, 1, 1, 128, 0, 8, 64,
                          None, None) == -4
    # zero tokens is a no-op
    assert lib.kv_scatter(None, None, 0, None, None, good, 64, good, 1, 1, 128, 0, 8, 64, None, None) == 0
    # unsupported head_dim
    assert lib.attn_prefill(good, good, 64, good, 1, 1, 128, 0, None, good, 1, 17, 32, 8, 96,
                            0.125, 1, good, good, None, None) == -3
    # Hq not a multiple of Hkv
    assert lib.attn_prefill(good, good, 64, good, 1, 1, 128, 0, None, good, 1, 17, 30, 8, 64,
                            0.125, 1, good, good, None, None) == -2
    # group size without a decode kernel
    assert lib.attn_decode(good, good, 64, good, 1, 1, 128, 0, None, good, 1, 96, 3, 64, 0.125,
                           64, good, 1 << 20, good, good, None, None) == -3
    # workspace too small (4 long contexts are split across workgroups)
    assert lib.attn_decode(good, good, 64, good, 4, 1, 1024, 0, None, good, 4, 32, 8, 64, 0.125,
                           16384, good, 16, good, good, None, None) == -5
    assert lib.attn_decode(good, good, 64, good, 4, 1, 1024, 0, None, good, 4, 32, 8, 64, 0.125,
                           16384, None, 0, good, good, None, None) == -1
    # page count overflow of int32 page ids
    assert lib.kv_scatter(good, good, 1, good, good, good, 1 << 31, good, 1, 1, 128, 0, 8, 64,
                          None, None) == -6
    assert lib.attn_prefill_dense(good, good, None, 1, 16, 4, 4, 64, 0.125, 1, good, good, None) == -1
    # chunked prefill needs q_lens
    assert lib.attn_prefill_chunk(good, good, 64, good, 1, 1, 128, 0, None, None, good, 1, 17, 32, 8,
                                  64, 0.125, 1, good, good, None, None) == -1
    assert lib.attn_prefill_chunk(good, good, 64, good, 1, 1, 128, 0, None, None, None, 0, 17, 32, 8,
                                  64, 0.125, 1, good, good, None, None) == 0


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_scale_outside_its_domain_is_rejected(scale):
    """The kernels take exp2(s * scale * log2 e - m) with -inf masks, which holds
    for a finite positive scale only: every attention call rejects any other
    value (PA_ERR_VALUE) before launching anything."""
    lib = pa.load()
    good = _fake()
    assert lib.attn_prefill(good, good, 64, good, 1, 1, 128, 0, None, good, 1, 17, 32, 8, 64,
                            scale, 1, good, good, None, None) == -8
    assert lib.attn_prefill_chunk(good, good, 64, good, 1, 1, 128, 0, None, good, good, 1, 17, 32, 8,
                                  64, scale, 1, good, good, None, None) == -8
    assert lib.attn_decode(good, good, 64, good, 1, 1, 128, 0, None, good, 1, 32, 8, 64, scale,
                           64, good, 1 << 20, good, good, None, None) == -8
    assert lib.attn_prefill_dense(good, good, good, 1, 16, 4, 4, 64, scale, 1, good, good, None) == -8
    assert lib.attn_backward_dense(good, good, good, good, good, good, 1, 16, 4, 4, 64, scale, 1,
                                   good, good, good, good, 1 << 20, None) == -8
    # the smallest and largest finite positive scales are accepted (zero-size no-op calls)
    for ok in (1e-30, 3.0e38):
        assert lib.attn_prefill_dense(None, None, None, 0, 16, 4, 4, 64, ok, 1, None, None, None) == 0


def test_noalloc_decode_host_checks():
    """attn_decode_noalloc checks its arguments like attn_decode before it looks
    anything up on the device; B == 0 is a no-op."""
    lib = pa.load()
    good = _fake()
    args = [good, good, 64, good, 1, 1, 128, 0, None, good, 1, 32, 8, 64, 0.125, 64, good, good,
            None, None]
    assert lib.attn_decode_noalloc(*args[:14], 0.0, *args[15:]) == -8
    assert lib.attn_decode_noalloc(None, *args[1:]) == -1
    assert lib.attn_decode_noalloc(*args[:11], 96, 3, *args[13:]) == -3
    assert lib.attn_decode_noalloc(*args[:10], 0, *args[11:]) == 0


def test_decode_append_host_checks():
    """attn_decode_append checks its arguments like attn_decode, then the new
    token's rows (present, 16-byte aligned); B == 0 is a no-op.  (Every call
    here is rejected on the host or does nothing: none launches.)"""
    lib = pa.load()
    good = _fake()
    args = [good, good, good, good, 64, good, 1, 1, 128, 0, None, good, 1, 32, 8, 64, 0.125, 64, None, 0,
            good, good, None, None]
    assert lib.attn_decode_append(*args[:16], 0.0, *args[17:]) == -8          # scale
    assert lib.attn_decode_append(args[0], None, *args[2:]) == -1              # k_new
    assert lib.attn_decode_append(*args[:2], None, *args[3:]) == -1            # v_new
    assert lib.attn_decode_append(args[0], ctypes.c_void_p(0x10002), *args[2:]) == -4
    assert lib.attn_decode_append(*args[:13], 96, 3, *args[15:]) == -3         # group 32
    assert lib.attn_decode_append(*args[:12], 0, *args[13:]) == 0              # B == 0


def test_prefill_append_host_checks():
    """attn_prefill_append checks its arguments like attn_prefill, then the
    prompt's K/V rows (present, 16-byte aligned); B == 0 or T == 0 is a no-op.
    (Every call here is rejected on the host or does nothing: none launches.)"""
    lib = pa.load()
    good = _fake()
    args = [good, good, good, good, 64, good, 1, 1, 128, 0, None, good, 1, 32, 32, 8, 64, 0.125, 1,
            good, good, None, None]
    assert lib.attn_prefill_append(*args[:17], 0.0, *args[18:]) == -8          # scale
    assert lib.attn_prefill_append(args[0], None, *args[2:]) == -1             # k
    assert lib.attn_prefill_append(*args[:2], None, *args[3:]) == -1           # v
    assert lib.attn_prefill_append(args[0], ctypes.c_void_p(0x10002), *args[2:]) == -4
    assert lib.attn_prefill_append(*args[:3], ctypes.c_void_p(0x10008), *args[4:]) == -4   # kv_cache
    assert lib.attn_prefill_append(*args[:14], 96, 3, *args[16:]) == -3        # group 32
    assert lib.attn_prefill_append(*args[:16], 72, *args[17:]) == -3           # head_dim 72
    assert lib.attn_prefill_append(*args[:9], 1, *args[10:]) == -2             # layer past n_layers
    assert lib.attn_prefill_append(*args[:12], 0, *args[13:]) == 0             # B == 0
    assert lib.attn_prefill_append(*args[:13], 0, *args[14:]) == 0             # T == 0


def _append(lib, **kw):
    good = _fake()
    a = dict(k=good, v=good, q_in=None, q_out=None, Hq=0, B=4, slot_ids=None, positions=good,
             cos_t=good, sin_t=good, max_pos=2048, kv_cache=good, n_pages=64, block_table=good,
             n_slots=4, n_layers=1, mbps=128, layer=0, free_pages=good, capacity=64, alloc=good, Hkv=8, d=64,
             err=None, stream=None)
    a.update(kw)
    return lib.kv_append(*a.values())


def test_append_release_host_checks():
    lib = pa.load()
    assert _append(lib, B=0, k=None, v=None, positions=None) == 0        # no-op
    assert _append(lib, alloc=None) == -1
    assert _append(lib, q_in=_fake()) == -1                              # q_in without q_out
    assert _append(lib, q_in=_fake(), q_out=_fake(), Hq=0) == -2
    assert _append(lib, d=72) == -3                                      # not a multiple of 16
    assert _append(lib, cos_t=_fake(0x10008)) == -4
    assert _append(lib, alloc=_fake(0x10002)) == -4
    assert _append(lib, max_pos=0) == -2
    assert _append(lib, layer=1) == -2
    assert _append(lib, capacity=-1) == -2
    good = _fake()
    assert lib.kv_release(None, 0, good, 4, 1, 128, good, 64, good, None, None) == 0
    assert lib.kv_release(None, 2, good, 4, 1, 128, good, 64, good, None, None) == -1
    assert lib.kv_release(good, 2, good, 4, 1, 128, good, -1, good, None, None) == -2
    assert lib.kv_release(good, 2, good, 4, 1, 128, good, 64, _fake(0x10001), None, None) == -4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pa, "_lib", None)
    with pytest.raises(ImportError):
        pa.load()
