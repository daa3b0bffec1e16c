"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

from nvfp4_compressed_sparse_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_nvfp4.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def _declared():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int|int32_t|int64_t|size_t|void|const char\*)\s+(mla_\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmla_nvfp4.so is not built; run __graft_entry__.build() first")
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(3).startswith(b"workspace")
    assert lib.mla_status_string(99) == b"unknown status"


def _quant(lib, **kw):
    a = dict(latent=0x1000, ls=512, rope=0x2000, rs=64, dtype=0, n=4, slots=0x3000, cache=0x4000,
             rows=100, stream=None)
    a.update(kw)
    return lib.mla_nvfp4_quantize_append(a["latent"], a["ls"], a["rope"], a["rs"], a["dtype"], a["n"],
                                         a["slots"], a["cache"], a["rows"], a["stream"])


def test_quantize_rejects_bad_arguments(lib):
    assert _quant(lib, dtype=7) == UNSUPPORTED
    assert _quant(lib, n=-1) == INVALID
    assert _quant(lib, n=0, latent=None, rope=None, slots=None, cache=None) == OK
    assert _quant(lib, latent=None) == INVALID
    assert _quant(lib, cache=None) == INVALID
    assert _quant(lib, latent=0x1001) == INVALID            # not 16-byte aligned
    assert _quant(lib, ls=256) == INVALID                   # stride below 512
    assert _quant(lib, rs=60) == INVALID
    assert lib.mla_fp8_quantize_append(0x1000, 512, 0x2000, 64, 0, 4, 0x3000, 0x4000, 10,
                                       ctypes.c_float(3.0), None) == INVALID   # not a power of two


def _decode(lib, **kw):
    a = dict(q=0x1000, qd=0, T=2, H=32, qst=32 * 576, qsh=576, cache=0x2000, fmt=0, rows=100,
             kv=1.0, idx=0x3000, topk=64, ist=64, bt=None, bs=64, bst=0, brows=0, bcols=0, ts=None,
             sm=0.04, out=0x4000, lse=0x5000, ws=0x6000, wsb=1 << 30, splits=1, stream=None)
    a.update(kw)
    return lib.mla_sparse_decode(a["q"], a["qd"], a["T"], a["H"], a["qst"], a["qsh"], a["cache"],
                                 a["fmt"], a["rows"], a["kv"], a["idx"], a["topk"], a["ist"], a["bt"],
                                 a["bs"], a["bst"], a["brows"], a["bcols"], a["ts"], a["sm"], a["out"], a["lse"],
                                 a["ws"], a["wsb"], a["splits"], a["stream"])


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, qd=5) == UNSUPPORTED
    assert _decode(lib, fmt=3) == UNSUPPORTED
    assert _decode(lib, H=24) == UNSUPPORTED
    assert _decode(lib, topk=0) == INVALID
    assert _decode(lib, topk=4096, ist=4096) == INVALID
    assert _decode(lib, T=-1) == INVALID
    assert _decode(lib, T=0, q=None, cache=None, idx=None, out=None) == OK
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, out=0x4004) == INVALID
    assert _decode(lib, qsh=500) == INVALID
    assert _decode(lib, qst=576) == INVALID                 # heads would overlap
    assert _decode(lib, ist=10) == INVALID
    assert _decode(lib, bt=0x7000) == INVALID               # block table without token_seq
    assert _decode(lib, bt=0x7000, ts=0x8000, brows=0, bcols=4, bst=4) == INVALID
    assert _decode(lib, splits=65) == INVALID
    # the launch grid (units rounded up to 8, times the splits) stays below 2^24 workgroups
    assert _decode(lib, T=1 << 21, splits=8) == INVALID
    assert _decode(lib, T=(1 << 21) - 8, splits=8, wsb=16) == WORKSPACE
    assert _decode(lib, fmt=1, kv=0.3) == INVALID
    assert _decode(lib, sm=float("inf")) == INVALID
    assert _decode(lib, ws=None) == WORKSPACE
    assert _decode(lib, wsb=16) == WORKSPACE


def test_workspace_size_arithmetic(lib):
    # one split: only the arrival state (64 bytes per (token, head group))
    # rounded up to 256 bytes
    assert lib.mla_sparse_decode_workspace_size(15, 32, 2048, 1) == 1024
    assert lib.mla_sparse_decode_workspace_size(100, 32, 2048, 1) == 6400
    # S splits add an lse block [T*G*S*32] f32 and an O block [T*G*S*32*512]
    # fp16, each part rounded to 256 bytes
    def expect(t, g, s):
        ctr = ((t * g * 64 + 255) // 256) * 256
        lse = ((t * g * s * 32 * 4 + 255) // 256) * 256
        return ctr + lse + t * g * s * 32 * 512 * 2
    assert lib.mla_sparse_decode_workspace_size(15, 32, 2048, 4) == expect(15, 1, 4)
    assert lib.mla_sparse_decode_workspace_size(100, 32, 2048, 4) == expect(100, 1, 4)
    assert lib.mla_sparse_decode_workspace_size(100, 64, 2048, 3) == expect(100, 2, 3)
    assert lib.mla_sparse_decode_workspace_size(15, 64, 2048, 1) == 2048      # 2 head groups
    assert lib.mla_sparse_decode_workspace_size(15, 24, 2048, 1) == 0
    assert lib.mla_sparse_decode_workspace_size(15, 32, 0, 1) == 0
    assert lib.mla_sparse_decode_workspace_size(15, 32, 2048, 99) == 0


def test_timing_query_without_a_timed_launch(lib):
    ms = ctypes.c_float(0.0)
    assert lib.mla_last_kernel_ms(None) == INVALID
    assert lib.mla_last_kernel_ms(ctypes.byref(ms)) == INVALID   # timing never enabled
    assert lib.mla_kernel_timing(0) == OK                         # disabling is always fine


def test_gather_dequant_rejects_bad_arguments(lib):
    f = lib.mla_nvfp4_gather_dequant_fp8
    assert f(0x1000, 10, 0x2000, 1, 8, 8, None, 64, 0, 0, 0, None, ctypes.c_float(0.0), 0x3000, 0x4000, None) == INVALID
    assert f(0x1000, 10, 0x2000, 1, 0, 8, None, 64, 0, 0, 0, None, ctypes.c_float(1.0), 0x3000, 0x4000, None) == INVALID
    assert f(0x1000, 10, 0x2000, 0, 8, 8, None, 64, 0, 0, 0, None, ctypes.c_float(1.0), 0x3000, 0x4000, None) == OK
    assert f(0x1000, 10, None, 1, 8, 8, None, 64, 0, 0, 0, None, ctypes.c_float(1.0), 0x3000, 0x4000, None) == INVALID


def test_noalloc_decode_rejects_bad_arguments_and_oversized_calls(lib):
    """Argument and scratch-size errors come back before any HIP call."""
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every case fails its checks first

    def call(T, H, topk, splits, fmt=0):
        return lib.mla_sparse_decode_noalloc(fake, 0, T, H, H * 576, 576, fake, fmt, 1000, 1.0,
                                             fake, topk, topk, None, 64, 0, 0, 0, None,
                                             0.1, fake, fake, splits, None)
    assert call(0, 32, 16, 1) == OK
    assert call(4, 33, 16, 1) == UNSUPPORTED
    assert call(4, 32, 0, 1) == INVALID
    assert call(4, 32, 16, 1, fmt=7) == UNSUPPORTED
    assert call(70000, 32, 2048, 1) == WORKSPACE        # more units than arrival states
    assert call(1000, 32, 2048, 2) == WORKSPACE         # partials past the scratch array
    assert call(300, 32, 2048, 4) == WORKSPACE


def test_indexer_rejects_bad_arguments(lib):
    """Host-side checks of mla_indexer_topk, before any HIP call."""
    fake = ctypes.c_void_p(1 << 20)

    def call(T=2, q_st=128, topk=16, out_st=16, max_ctx=100, base=fake, bt=None, seq=None, ws_bytes=1 << 30):
        return lib.mla_indexer_topk(fake, q_st, fake, 1000, T, fake, max_ctx, base, bt, 64, 4, 2, 4, seq,
                                    topk, fake, out_st, fake, ws_bytes, None)
    assert call(T=0) == OK
    assert call(topk=0) == INVALID and call(topk=2049) == INVALID
    assert call(q_st=120) == INVALID and call(q_st=136) == INVALID      # stride: >= 128, multiple of 16
    assert call(out_st=8) == INVALID
    assert call(base=None) == INVALID                                   # rows need a base or a table
    assert call(base=None, bt=fake) == INVALID                          # a table needs token_seq
    assert call(max_ctx=-1) == INVALID
    assert call(ws_bytes=16) == WORKSPACE
    r = lambda x: (x + 255) // 256 * 256

    def layout(T, max_ctx):   # histograms, candidate counts, keys, candidate keys and positions, two bitmaps
        ks, wsd = (max_ctx + 1) // 2 * 2, ((max_ctx + 31) // 32 + 3) // 4 * 4
        return r(T * 4096 * 4) + r(T * 4) + 2 * r(T * ks * 8) + r(T * ks * 4) + r(T * wsd * 4) + T * wsd * 4
    need = lib.mla_indexer_workspace_size(2, 100)
    assert need == layout(2, 100)
    assert lib.mla_indexer_workspace_size(3, 101) == layout(3, 101)


def test_gather_probe_rejects_bad_arguments(lib):
    """Host-side checks of mla_gather_probe, before any HIP call."""
    fake = ctypes.c_void_p(1 << 20)

    def call(rows_n=10, row_bytes=352, cache=fake, rows=fake, sink=fake, cache_rows=100):
        return lib.mla_gather_probe(cache, cache_rows, row_bytes, rows, rows_n, sink, None)
    assert call(rows_n=0) == OK
    assert call(row_bytes=350) == INVALID and call(row_bytes=0) == INVALID
    assert call(rows_n=-1) == INVALID and call(cache_rows=-1) == INVALID
    assert call(rows=None) == INVALID and call(sink=None) == INVALID
    assert call(cache=ctypes.c_void_p((1 << 20) + 8)) == INVALID     # cache not 16-byte aligned
    assert call(rows_n=1 << 31) == INVALID


def test_merge_polls_setting(lib):
    prev = lib.mla_sparse_decode_set_merge_polls(7)
    try:
        assert prev >= 0
        assert lib.mla_sparse_decode_set_merge_polls(0) == 7
        assert lib.mla_sparse_decode_set_merge_polls(-3) == -1      # rejected, unchanged
        assert lib.mla_sparse_decode_set_merge_polls(5) == 0
    finally:
        lib.mla_sparse_decode_set_merge_polls(prev)


def test_launch_sizer_choices(lib):
    # (no GPU here: the sizer assumes MI355X's 256 CUs in 8 XCDs)
    # S = CUs / units, capped at topk / 256 and 64; one split fewer where
    # that puts every unit's splits on one XCD in one round of workgroups
    assert lib.mla_sparse_decode_num_splits(1, 16, 256) == 1        # tiny
    assert lib.mla_sparse_decode_num_splits(15, 32, 2048) == 8      # decode15 (topk cap)
    assert lib.mla_sparse_decode_num_splits(35, 32, 2048) == 6      # padded35: 7 would not group
    assert lib.mla_sparse_decode_num_splits(128, 32, 2048) == 2     # batch128
    assert lib.mla_sparse_decode_num_splits(4096, 32, 2048) == 1    # prefill4k
    assert lib.mla_sparse_decode_num_splits(40, 32, 2048) == 6      # 6 groups already
    assert lib.mla_sparse_decode_num_splits(1, 32, 2048) == 8
