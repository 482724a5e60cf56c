"""The C-ABI library loads on the CPU, exports every symbol include/lca.h
declares, and rejects bad calls before touching the GPU (no compute calls
are made here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "lca.h")
LIB = os.path.join(ROOT, "long_context_compressed_append_amd", "liblca.so")


def _lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return C.CDLL(LIB)


def declared_symbols():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lca_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = _lib()
    syms = declared_symbols()
    assert {"lca_compress_append", "lca_indexer_topk", "lca_csa_attend", "lca_hca_attend"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_abi_version():
    L = _lib()
    assert L.lca_abi_version() == 3


def _layer(**kw):
    from long_context_compressed_append_amd import LcaLayerStruct
    s = LcaLayerStruct()
    s.batch, s.ratio, s.window, s.ring, s.has_indexer, s.max_blocks = 1, 4, 16, 64, 0, 16
    fake = 0x10000   # aligned, never dereferenced: validation fails first
    for f in ("seq_len", "sync", "nope", "rope", "kv_scale", "ring_kv", "ring_gate", "pos_bias"):
        setattr(s, f, fake)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


@pytest.mark.parametrize("kw,code", [
    (dict(ratio=3), -2),            # not a power of two
    (dict(ratio=256), -2),
    (dict(batch=0), -1),
    (dict(ring=8), -3),             # ring < window
    (dict(seq_len=None), -1),
    (dict(nope=0x10001), -1),       # misaligned
    (dict(has_indexer=1), -1),      # indexer planes missing
    (dict(len_min=5, len_max=2), -1),
    # paged entry planes
    (dict(page_table=0x10000), -1),                                           # table without pages
    (dict(page_blocks=32, max_blocks=128, page_table=0x10000, pool_pages=4), -2),    # below 64
    (dict(page_blocks=96, max_blocks=192, page_table=0x10000, pool_pages=4), -2),    # not a power of two
    (dict(page_blocks=64, max_blocks=100, page_table=0x10000, pool_pages=4), -1),    # MB not a multiple
    (dict(page_blocks=64, max_blocks=128, page_table=None, pool_pages=4), -1),
    (dict(page_blocks=64, max_blocks=128, page_table=0x10002, pool_pages=4), -1),    # misaligned table
    (dict(page_blocks=64, max_blocks=128, page_table=0x10000, pool_pages=0), -1),
    (dict(page_blocks=65536, max_blocks=65536, page_table=0x10000, pool_pages=1 << 15), -2),  # pool >= 2^31
])
def test_layer_validation(kw, code):
    L = _lib()
    L.lca_last_error.restype = C.c_char_p
    s = _layer(**kw)
    rc = L.lca_compress_append(C.byref(s), C.c_void_p(0x10000), C.c_void_p(0x10000), None, None, 1, None)
    assert rc == code, L.lca_last_error()
    assert L.lca_last_error()


def test_call_validation():
    L = _lib()
    L.lca_last_error.restype = C.c_char_p
    s = _layer()
    p = C.c_void_p(0x10000)
    # ring too small for the append
    assert L.lca_compress_append(C.byref(s), p, p, None, None, 60, None) == -3
    # capacity: 16 blocks * 4 = 64 tokens
    s2 = _layer(ring=200)
    assert L.lca_compress_append(C.byref(s2), p, p, None, None, 100, None) == -3
    # indexer on an HCA layer
    assert L.lca_indexer_topk(C.byref(s), p, p, 1, 4, 8, p, p, C.c_size_t(1 << 20), None) == -1
    # n_q beyond the shortest row
    assert L.lca_hca_attend(C.byref(s), p, 1, 16, C.c_float(0.04), p, None, C.c_size_t(0), None) == -1
    s3 = _layer(len_min=10, len_max=10)
    # H out of range
    assert L.lca_hca_attend(C.byref(s3), p, 1, 129, C.c_float(0.04), p, None, C.c_size_t(0), None) == -2
    # k out of range
    assert L.lca_csa_attend(C.byref(s3), p, 1, 16, p, 0, C.c_float(0.04), p, None, C.c_size_t(0),
                            None) == -2
    # n == 0 is a no-op
    assert L.lca_compress_append(C.byref(s), p, p, None, None, 0, None) == 0
    # a valid paged layer passes validation
    s4 = _layer(page_blocks=64, max_blocks=128, page_table=0x10000, pool_pages=3)
    assert L.lca_compress_append(C.byref(s4), p, p, None, None, 0, None) == 0, L.lca_last_error()


def test_workspace_queries_are_pure():
    L = _lib()
    L.lca_attend_workspace.restype = C.c_size_t
    L.lca_indexer_workspace.restype = C.c_size_t
    s = _layer(len_min=131072, len_max=131072, max_blocks=33000, has_indexer=1)
    n = L.lca_indexer_workspace(C.byref(s), 1, 16, 512)
    assert n >= 4 * 32768
    a = L.lca_attend_workspace(C.byref(s), 1, 64, 512)
    assert a % 4 == 0


def test_indexer_layout_matches_the_workspace():
    """The layout query (host only): candidate segments for a decode query
    (the selection in the scoring launch), full key rows when the separate
    selection is forced, candidate lists for a prefill chunk, every region
    inside the workspace size."""
    L = _lib()
    L.lca_indexer_workspace.restype = C.c_size_t
    L.lca_indexer_layout.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int64)]
    L.lca_set_tuning.argtypes = [C.c_char_p, C.c_int32]
    out = (C.c_int64 * 8)()
    # decode: one query per row, per-workgroup candidate segments
    s = _layer(batch=4, len_min=131072, len_max=131072, max_blocks=33000, has_indexer=1)
    assert L.lca_indexer_layout(C.byref(s), 1, 16, 512, out) == 0
    stride, keys, kind, zero, counts, segs, span = out[0], out[1], out[2], out[3], out[4], out[5], out[7]
    assert stride >= 32768 and stride % 64 == 0 and kind == 2
    assert zero == keys and zero >= 4 * 4096 * 4 + 4 * 4  # row counters, then the histograms
    assert segs * span >= 32768 and span % 1024 == 0
    total = L.lca_indexer_workspace(C.byref(s), 1, 16, 512)
    assert keys + 4 * stride * 8 <= counts and counts + 4 * segs * 4 <= total
    # the same with the separate selection: full key rows after the histograms
    assert L.lca_set_tuning(b"LCA_TOPK_FUSED", 0) == 0
    try:
        assert L.lca_indexer_layout(C.byref(s), 1, 16, 512, out) == 0
        stride, keys, kind, zero = out[0], out[1], out[2], out[3]
        assert kind == 0 and keys == zero == 4 * 4096 * 4
        assert keys + 4 * stride * 4 <= L.lca_indexer_workspace(C.byref(s), 1, 16, 512)
    finally:
        L.lca_set_tuning(b"LCA_TOPK_FUSED", -1)
    # prefill chunk: 4096 queries in one row, candidate lists
    s = _layer(batch=1, len_min=266240, len_max=266240, max_blocks=66624, has_indexer=1)
    n_q = 4096
    assert L.lca_indexer_layout(C.byref(s), n_q, 16, 512, out) == 0
    stride, keys, cand, counts, lists, waves, span = out[0], out[1], out[2], out[4], out[5], out[6], out[7]
    assert cand == 1 and waves == 8 and lists % (32 * waves) == 0
    chunks = lists // (32 * waves)
    assert chunks * span >= 266240 // 4 and span % 1024 == 0
    total = L.lca_indexer_workspace(C.byref(s), n_q, 16, 512)
    assert keys + n_q * stride * 8 <= counts          # (key, visit) pairs, then the list lengths
    assert counts + n_q * lists * 4 <= total
    # errors
    assert L.lca_indexer_layout(C.byref(s), 0, 16, 512, out) == -1
    assert L.lca_indexer_layout(C.byref(s), 1, 16, 512, None) == -1


def test_set_tuning_names():
    L = _lib()
    L.lca_set_tuning.argtypes = [C.c_char_p, C.c_int32]
    L.lca_last_error.restype = C.c_char_p
    for name in ("LCA_SCORE_TILE", "LCA_TOPK_CAND", "LCA_TOPK_SLICED", "LCA_TOPK_FUSED", "LCA_SCORE_CPW",
                 "LCA_ATTEND_SPLITS"):
        assert L.lca_set_tuning(name.encode(), 1) == 0
        assert L.lca_set_tuning(name.encode(), -1) == 0       # back to automatic
    assert L.lca_set_tuning(b"LCA_NO_SUCH_KNOB", 1) == -1
    assert b"unknown" in L.lca_last_error()
    assert L.lca_set_tuning(None, 1) == -1
