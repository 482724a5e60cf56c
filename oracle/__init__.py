"""ctypes wrapper over the plain CPU oracle (liblca_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Arrays are numpy;
a layer is the dict of planes built by synth.layers (the same plane layout the
HIP library uses).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lca_oracle.c")
LIB = os.path.join(HERE, "liblca_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", "-o", LIB + ".tmp", SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = C.CDLL(LIB)
        _setup(_lib)
    return _lib


P = C.c_void_p


class OrcLayer(C.Structure):
    _fields_ = [("batch", C.c_int32), ("ratio", C.c_int32), ("window", C.c_int32),
                ("ring", C.c_int32), ("has_indexer", C.c_int32), ("page_blocks", C.c_int32),
                ("max_blocks", C.c_int64),
                ("seq_len", P), ("nope", P), ("rope", P), ("kv_scale", P),
                ("idx_code", P), ("idx_scale", P), ("ring_kv", P), ("ring_gate", P),
                ("ring_ikey", P), ("ring_igate", P), ("pos_bias", P), ("ipos_bias", P),
                ("page_table", P), ("pool_pages", C.c_int64)]


def _setup(L):
    L.orc_bf16_value.restype = C.c_double
    L.orc_bf16_value.argtypes = [C.c_uint16]
    L.orc_bf16_encode.restype = C.c_uint16
    L.orc_bf16_encode.argtypes = [C.c_float]
    L.orc_e4m3_value.restype = C.c_double
    L.orc_e4m3_value.argtypes = [C.c_uint8]
    L.orc_e4m3_encode.restype = C.c_uint8
    L.orc_e4m3_encode.argtypes = [C.c_float]
    L.orc_e2m1_value.restype = C.c_double
    L.orc_e2m1_value.argtypes = [C.c_uint8]
    L.orc_e2m1_encode.restype = C.c_uint8
    L.orc_e2m1_encode.argtypes = [C.c_float]
    L.orc_e8m0_value.restype = C.c_double
    L.orc_e8m0_value.argtypes = [C.c_uint8]
    L.orc_fp8_group_quant.argtypes = [P, P, P]
    L.orc_mxfp4_quant.argtypes = [P, P, P]
    L.orc_pool_f32.argtypes = [C.c_int, C.c_int, P, C.c_long, P, C.c_long, P, P]
    L.orc_pool_f64.argtypes = [C.c_int, C.c_int, P, C.c_long, P, C.c_long, P, P]
    L.orc_make_entry.argtypes = [P, P, P, P]
    L.orc_make_idx.argtypes = [P, P, P]
    L.orc_compress_append.argtypes = [C.POINTER(OrcLayer), P, P, P, P, C.c_int]
    L.orc_entry_index.restype = C.c_long
    L.orc_entry_index.argtypes = [C.POINTER(OrcLayer), C.c_int, C.c_long]
    L.orc_index_score.restype = C.c_float
    L.orc_index_score.argtypes = [P, P, P, C.c_int, P, P, C.POINTER(C.c_int)]
    L.orc_topk_select.argtypes = [P, C.c_int, C.c_int, P]
    L.orc_indexer_topk.argtypes = [C.POINTER(OrcLayer), P, P, C.c_int, C.c_int, C.c_int, P, C.c_int]
    L.orc_indexer_scores.argtypes = [C.POINTER(OrcLayer), C.c_int, C.c_int, C.c_int, P, P, C.c_int,
                                     P, C.POINTER(C.c_int)]
    L.orc_attend_keys.argtypes = [P, C.c_int, C.c_int, P, C.c_double, P]
    L.orc_csa_attend.argtypes = [C.POINTER(OrcLayer), P, C.c_int, C.c_int, P, C.c_int, C.c_float, P,
                                 C.c_int]
    L.orc_hca_attend.argtypes = [C.POINTER(OrcLayer), P, C.c_int, C.c_int, C.c_float, P, C.c_int]


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be C-contiguous"
    return a.ctypes.data


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def nthreads_default():
    """The threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (a job's share of a shared host)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


# ---------------------------------------------------------------- formats

def bf16_value(b):
    return lib().orc_bf16_value(int(b))


def bf16_encode(x):
    return lib().orc_bf16_encode(float(x))


def e4m3_value(c):
    return lib().orc_e4m3_value(int(c))


def e4m3_encode(x):
    return lib().orc_e4m3_encode(float(x))


def e2m1_value(c):
    return lib().orc_e2m1_value(int(c))


def e2m1_encode(x):
    return lib().orc_e2m1_encode(float(x))


def e8m0_value(e):
    return lib().orc_e8m0_value(int(e))


def fp8_group_quant(y):
    y = _f32(y)
    assert y.size == 64
    codes = np.zeros(64, np.uint8)
    s = np.zeros(1, np.float32)
    lib().orc_fp8_group_quant(_p(y), _p(codes), _p(s))
    return codes, float(s[0])


def mxfp4_quant(y):
    y = _f32(y)
    assert y.size == 32
    packed = np.zeros(16, np.uint8)
    e = np.zeros(1, np.uint8)
    lib().orc_mxfp4_quant(_p(y), _p(packed), _p(e))
    return packed, int(e[0])


def make_entry(y):
    y = _f32(y)
    nope = np.zeros(448, np.uint8)
    rope = np.zeros(64, np.uint16)
    sc = np.zeros(8, np.float32)
    lib().orc_make_entry(_p(y), _p(nope), _p(rope), _p(sc))
    return nope, rope, sc


def make_idx(y):
    y = _f32(y)
    code = np.zeros(32, np.uint8)
    e = np.zeros(2, np.uint8)
    lib().orc_make_idx(_p(y), _p(code), _p(e))
    return code, e


# ---------------------------------------------------------------- compressor

def pool(x, z, bias, double=False):
    """x [m][C] float32 (raw values), z [m][C] gate logits, bias [m][C]."""
    x, z, bias = _f32(x), _f32(z), _f32(bias)
    m, Cc = x.shape
    if double:
        y = np.zeros(Cc, np.float64)
        lib().orc_pool_f64(m, Cc, _p(x), Cc, _p(z), Cc, _p(bias), _p(y))
    else:
        y = np.zeros(Cc, np.float32)
        lib().orc_pool_f32(m, Cc, _p(x), Cc, _p(z), Cc, _p(bias), _p(y))
    return y


def layer_struct(L):
    s = OrcLayer()
    s.batch, s.ratio, s.window, s.ring = L["batch"], L["ratio"], L["window"], L["ring"]
    s.has_indexer, s.max_blocks = L["has_indexer"], L["max_blocks"]
    s.page_blocks, s.pool_pages = int(L.get("page_blocks", 0)), int(L.get("pool_pages", 0))
    for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
              "ring_gate", "ring_ikey", "ring_igate", "pos_bias", "ipos_bias", "page_table"):
        a = L.get(f)
        setattr(s, f, _p(a) if a is not None and a.size else None)
    if s.page_blocks:
        assert L["page_table"].dtype == np.int32 and L["page_table"].flags["C_CONTIGUOUS"]
    return s


def compress_append(L, kv, gate, ikey=None, igate=None):
    """Mutates the layer dict L in place, like the library call."""
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    B, n = kv.shape[0], kv.shape[1]
    assert B == L["batch"]
    gate = _f32(gate)
    ikey = _f32(ikey) if ikey is not None else None
    igate = _f32(igate) if igate is not None else None
    s = layer_struct(L)
    rc = lib().orc_compress_append(C.byref(s), _p(kv), _p(gate), _p(ikey), _p(igate), n)
    if rc:
        raise RuntimeError(f"oracle compress_append failed ({rc})")


# ---------------------------------------------------------------- indexer

def index_score(qcode, qe, w, kcode, ke):
    qcode = np.ascontiguousarray(qcode, np.uint8)
    qe = np.ascontiguousarray(qe, np.uint8)
    w = _f32(w)
    kcode = np.ascontiguousarray(kcode, np.uint8)
    ke = np.ascontiguousarray(ke, np.uint8)
    inexact = C.c_int(0)
    s = lib().orc_index_score(_p(qcode), _p(qe), _p(w), int(w.size), _p(kcode), _p(ke),
                              C.byref(inexact))
    return s, bool(inexact.value)


def topk_select(scores, k):
    scores = _f32(scores)
    out = np.zeros(k, np.int32)
    lib().orc_topk_select(_p(scores), int(scores.size), int(k), _p(out))
    return out


def indexer_scores(L, row, qi, n_q, iq, iw):
    """Scores of query qi of row `row`: iq [rows][n_q][H][64] and iw
    [rows][n_q][H] hold that row (row < rows)."""
    iq, iw = _f32(iq), _f32(iw)
    H = iw.shape[-1]
    if not (0 <= row < iq.shape[0] and iq.shape[:3] == iw.shape and iq.shape[1] == n_q and 0 <= qi < n_q):
        raise ValueError(f"indexer_scores: row {row}, query {qi} not in iq {iq.shape} / iw {iw.shape}")
    s = layer_struct(L)
    out = np.zeros(L["max_blocks"] + 1, np.float32)
    nv = C.c_int(0)
    rc = lib().orc_indexer_scores(C.byref(s), row, qi, n_q, _p(iq), _p(iw), H, _p(out), C.byref(nv))
    if rc:
        raise RuntimeError(f"oracle indexer_scores failed ({rc})")
    return out[: nv.value]


def indexer_topk(L, iq, iw, k, nthreads=None):
    iq, iw = _f32(iq), _f32(iw)
    B, n_q, H = iw.shape
    out = np.zeros((B, n_q, k), np.int32)
    s = layer_struct(L)
    rc = lib().orc_indexer_topk(C.byref(s), _p(iq), _p(iw), n_q, H, k, _p(out),
                                nthreads or nthreads_default())
    if rc:
        raise RuntimeError(f"oracle indexer_topk failed ({rc})")
    return out


# ---------------------------------------------------------------- attention

def attend_keys(q, keys, scale):
    q = np.ascontiguousarray(q, np.uint16)
    keys = np.ascontiguousarray(keys, np.float64)
    H = q.shape[0]
    out = np.zeros((H, 512), np.float32)
    lib().orc_attend_keys(_p(q), H, int(keys.shape[0]), _p(keys), float(scale), _p(out))
    return out


def csa_attend(L, q, topk, scale, nthreads=None):
    q = np.ascontiguousarray(q, np.uint16)
    topk = np.ascontiguousarray(topk, np.int32)
    B, n_q, H, _ = q.shape
    k = topk.shape[-1]
    out = np.zeros((B, n_q, H, 512), np.float32)
    s = layer_struct(L)
    rc = lib().orc_csa_attend(C.byref(s), _p(q), n_q, H, _p(topk), k, float(scale), _p(out),
                              nthreads or nthreads_default())
    if rc:
        raise RuntimeError(f"oracle csa_attend failed ({rc})")
    return out


def hca_attend(L, q, scale, nthreads=None):
    q = np.ascontiguousarray(q, np.uint16)
    B, n_q, H, _ = q.shape
    out = np.zeros((B, n_q, H, 512), np.float32)
    s = layer_struct(L)
    rc = lib().orc_hca_attend(C.byref(s), _p(q), n_q, H, float(scale), _p(out),
                              nthreads or nthreads_default())
    if rc:
        raise RuntimeError(f"oracle hca_attend failed ({rc})")
    return out


def row_view(L, row):
    """A one-row layer dict sharing memory with row `row` of L (a paged
    layer's view keeps the whole page pool and the row's page table)."""
    V = dict(L)
    V["batch"] = 1
    V["seq_len"] = L["seq_len"][row:row + 1]
    planes = ["ring_kv", "ring_gate", "ring_ikey", "ring_igate"]
    if L.get("page_blocks", 0):
        V["page_table"] = L["page_table"][row:row + 1]
    else:
        planes += ["nope", "rope", "kv_scale", "idx_code", "idx_scale"]
    for f in planes:
        V[f] = L[f][row:row + 1]
    return V


def entry_index(L, row, b):
    """Where entry b of row `row` lives in L's entry planes (-1: unmapped page)."""
    s = layer_struct(L)
    return int(lib().orc_entry_index(C.byref(s), int(row), int(b)))
