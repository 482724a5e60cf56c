"""Python binding of liblca.so (MI355X / gfx950 compressed long-context attention).

Argument marshalling only: every step of the path runs in the HIP kernels of
liblca.so, called through its C ABI (include/lca.h) with plain device
pointers and the current HIP stream.  PyTorch provides device memory and
streams.  There is no CPU fallback: if the library is missing or the GPU is
absent, the calls raise.

    import long_context_compressed_append_amd as lca
    layer = lca.Layer(batch=32, ratio=4, window=128, ring=256, has_indexer=True,
                      max_blocks=33000)
    lca.compress_append(layer, kv, gate, ikey, igate)   # appends n tokens per row
    topk = lca.indexer_topk(layer, iq, iw, k=512)
    out = lca.csa_attend(layer, q, topk)
    out = lca.hca_attend(hca_layer, q)
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblca.so")

KV, NOPE, ROPE, IDX = 512, 448, 64, 64
ERRORS = {0: "LCA_OK", -1: "LCA_EINVAL", -2: "LCA_EUNSUPPORTED", -3: "LCA_ECAPACITY",
          -4: "LCA_EWORKSPACE", -5: "LCA_EHIP"}
STATUS_COMPRESS_CAPACITY, STATUS_INDEXER_CAPACITY, STATUS_ATTEND_CAPACITY, STATUS_FP16_RANGE = 1, 2, 4, 8
STATUS_PAGE = 16


class LcaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


P = C.c_void_p


class LcaLayerStruct(C.Structure):
    _fields_ = [("batch", C.c_int32), ("ratio", C.c_int32), ("window", C.c_int32),
                ("ring", C.c_int32), ("has_indexer", C.c_int32), ("page_blocks", C.c_int32),
                ("max_blocks", C.c_int64), ("len_min", C.c_int64), ("len_max", C.c_int64),
                ("seq_len", P), ("sync", P), ("nope", P), ("rope", P), ("kv_scale", P),
                ("idx_code", P), ("idx_scale", P), ("ring_kv", P), ("ring_gate", P),
                ("ring_ikey", P), ("ring_igate", P), ("pos_bias", P), ("ipos_bias", P),
                ("page_table", P), ("pool_pages", C.c_int64)]


_lib = None


def lib():
    """Load liblca.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "or python long_context_compressed_append_amd/build.py")
        L = C.CDLL(LIB_PATH)
        LP = C.POINTER(LcaLayerStruct)
        L.lca_abi_version.restype = C.c_int
        L.lca_last_error.restype = C.c_char_p
        L.lca_compress_append.argtypes = [LP, P, P, P, P, C.c_int32, P]
        L.lca_indexer_workspace.restype = C.c_size_t
        L.lca_indexer_workspace.argtypes = [LP, C.c_int32, C.c_int32, C.c_int32]
        L.lca_indexer_layout.argtypes = [LP, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int64)]
        L.lca_indexer_topk.argtypes = [LP, P, P, C.c_int32, C.c_int32, C.c_int32, P, P, C.c_size_t, P]
        L.lca_indexer_topk_noalloc.argtypes = [LP, P, P, C.c_int32, C.c_int32, C.c_int32, P, P]
        L.lca_decode_append_workspace.restype = C.c_size_t
        L.lca_decode_append_workspace.argtypes = [LP, C.c_int32, C.c_int32]
        L.lca_decode_append_topk.argtypes = [LP, P, P, P, P, P, P, C.c_int32, C.c_int32, P, P, C.c_size_t, P]
        L.lca_attend_workspace.restype = C.c_size_t
        L.lca_attend_workspace.argtypes = [LP, C.c_int32, C.c_int32, C.c_int32]
        L.lca_csa_attend.argtypes = [LP, P, C.c_int32, C.c_int32, P, C.c_int32, C.c_float, P, P,
                                     C.c_size_t, P]
        L.lca_hca_attend.argtypes = [LP, P, C.c_int32, C.c_int32, C.c_float, P, P, C.c_size_t, P]
        L.lca_set_tuning.argtypes = [C.c_char_p, C.c_int32]
        L.lca_timing_begin.argtypes = [C.c_char_p]
        L.lca_timing_end.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int64)]
        L.lca_timing_durations.argtypes = [C.POINTER(C.c_float), C.c_int64, C.POINTER(C.c_int64)]
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise LcaError(rc, lib().lca_last_error().decode(errors="replace"))


def _stream():
    return P(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _dev(t, dtype, shape=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


class Layer:
    """One layer's cache in device memory (plane layout of include/lca.h).

    Planes are torch tensors on `device`; `from_host` uploads numpy planes of
    the same layout (the dict built by synth.layers).  With page_blocks > 0
    the entry planes are a pool of pool_pages pages, [pool_pages *
    page_blocks][...], and page_table [B][max_blocks / page_blocks] (int32,
    -1 = unmapped) places each row's entries in it."""

    PLANES = ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
              "ring_gate", "ring_ikey", "ring_igate")

    def __init__(self, batch, ratio, window, ring, has_indexer, max_blocks, device="cuda",
                 pos_bias=None, ipos_bias=None, lengths=None, page_blocks=0, pool_pages=0):
        self.batch, self.ratio, self.window, self.ring = int(batch), int(ratio), int(window), int(ring)
        self.has_indexer, self.max_blocks = int(bool(has_indexer)), int(max_blocks)
        self.page_blocks, self.pool_pages = int(page_blocks), int(pool_pages)
        B, MB, R = self.batch, self.max_blocks, self.ring
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.seq_len = z((B,), torch.int32)
        self.sync = z((4,), torch.int32)
        ent = (B, MB)                         # entry planes: per row, or one pool
        self.page_table = None
        self.planes = self.PLANES
        if self.page_blocks:
            ent = (self.pool_pages * self.page_blocks,)
            self.page_table = torch.full((B, MB // self.page_blocks), -1, dtype=torch.int32, device=device)
            self.planes = self.PLANES + ("page_table",)
        self.nope = z(ent + (NOPE,), torch.uint8)
        self.rope = z(ent + (ROPE,), torch.int16)
        self.kv_scale = z(ent + (8,), torch.float32)
        hi = self.has_indexer
        self.idx_code = z(ent + (32,), torch.uint8) if hi else None
        self.idx_scale = z(ent + (2,), torch.uint8) if hi else None
        self.ring_kv = z((B, R, KV), torch.int16)
        self.ring_gate = z((B, R, KV), torch.float32)
        self.ring_ikey = z((B, R, IDX), torch.float32) if hi else None
        self.ring_igate = z((B, R, IDX), torch.float32) if hi else None
        self.pos_bias = (torch.as_tensor(pos_bias, dtype=torch.float32).to(device).contiguous()
                         if pos_bias is not None else z((self.ratio, KV), torch.float32))
        self.ipos_bias = None
        if hi:
            self.ipos_bias = (torch.as_tensor(ipos_bias, dtype=torch.float32).to(device).contiguous()
                              if ipos_bias is not None else z((self.ratio, IDX), torch.float32))
        self.len_min = self.len_max = 0
        if lengths is not None:
            self.set_lengths(lengths)
        self._ws = {}

    @classmethod
    def from_host(cls, L, device="cuda"):
        """Upload a numpy plane dict (synth.layers layout)."""
        lay = cls(L["batch"], L["ratio"], L["window"], L["ring"], L["has_indexer"], L["max_blocks"],
                  device=device, pos_bias=L["pos_bias"], ipos_bias=L.get("ipos_bias"),
                  page_blocks=L.get("page_blocks", 0), pool_pages=L.get("pool_pages", 0))
        lay.upload(L)
        return lay

    def upload(self, L):
        import numpy as np
        for f in self.planes:
            t = getattr(self, f)
            if t is None:
                continue
            a = np.ascontiguousarray(L[f])
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            t.copy_(torch.from_numpy(a).to(t.device))
        self.len_min = int(L["seq_len"].min())
        self.len_max = int(L["seq_len"].max())

    def download(self):
        """Planes back to host numpy (uint16 for bf16 planes)."""
        import numpy as np
        out = dict(batch=self.batch, ratio=self.ratio, window=self.window, ring=self.ring,
                   has_indexer=self.has_indexer, max_blocks=self.max_blocks)
        if self.page_blocks:
            out.update(page_blocks=self.page_blocks, pool_pages=self.pool_pages)
        for f in self.planes:
            t = getattr(self, f)
            if t is None:
                continue
            a = t.cpu().numpy()
            if a.dtype == np.int16:
                a = a.view(np.uint16)
            out[f] = a
        out["pos_bias"] = self.pos_bias.cpu().numpy()
        out["ipos_bias"] = self.ipos_bias.cpu().numpy() if self.ipos_bias is not None else None
        return out

    def status(self):
        """The layer's status bits (LCA_STATUS_*: 1 compressor capacity,
        2 indexer capacity, 4 attention capacity, 8 fp16 range, 16 unmapped
        page), as left by the work the stream has run so far."""
        return int(self.sync[1].item()) & 0xFFFFFFFF

    def clear_status(self):
        self.sync[1].zero_()

    def set_lengths(self, lengths):
        lengths = torch.as_tensor(lengths, dtype=torch.int32)
        self.seq_len.copy_(lengths.to(self.seq_len.device))
        self.len_min, self.len_max = int(lengths.min()), int(lengths.max())

    def struct(self):
        s = LcaLayerStruct()
        s.batch, s.ratio, s.window, s.ring = self.batch, self.ratio, self.window, self.ring
        s.has_indexer, s.page_blocks, s.max_blocks = self.has_indexer, self.page_blocks, self.max_blocks
        s.len_min, s.len_max = self.len_min, self.len_max
        s.pool_pages = self.pool_pages
        for f in ("seq_len", "sync", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
                  "ring_gate", "ring_ikey", "ring_igate", "pos_bias", "ipos_bias", "page_table"):
            t = getattr(self, f)
            setattr(s, f, t.data_ptr() if t is not None else None)
        return s

    def workspace(self, nbytes, kind="attend"):
        """A cached, zero-initialised device workspace of at least nbytes, one
        per kind.  The indexer's kind is ("indexer", B * n_q): its workspace
        starts with one zeroed histogram per query, which every call leaves
        zeroed, followed by data of that call; a call with more queries would
        find that data where its own histograms lie, so each query count
        keeps a workspace of its own."""
        if nbytes == 0:
            return None
        ws = self._ws.get(kind)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(int(nbytes), dtype=torch.uint8, device=self.seq_len.device)
            self._ws[kind] = ws
        return ws

    def indexer_workspace(self, n_q, nbytes=0):
        """The indexer workspace for calls with n_q queries per row."""
        return self.workspace(nbytes, ("indexer", self.batch * int(n_q))) if nbytes else \
            self._ws.get(("indexer", self.batch * int(n_q)))


def abi_version():
    return lib().lca_abi_version()


def set_tuning(name, value=None):
    """Force a kernel choice (lca_set_tuning); None or a negative value
    restores the automatic choice."""
    _check(lib().lca_set_tuning(name.encode(), -1 if value is None else int(value)))


TUNING_NAMES = ("LCA_SCORE_TILE", "LCA_TOPK_CAND", "LCA_TOPK_SLICED", "LCA_TOPK_FUSED", "LCA_SCORE_CPW",
                "LCA_ATTEND_SPLITS")


def compress_append(layer: Layer, kv, gate, ikey=None, igate=None):
    """Append n tokens to every row.  kv int16/bf16 bits [B][n][512], gate fp32
    [B][n][512], ikey/igate fp32 [B][n][64] (indexer layers)."""
    B = layer.batch
    if kv.dtype == torch.bfloat16:
        kv = kv.view(torch.int16)
    n = kv.shape[1]
    _dev(kv, torch.int16, (B, n, KV), "kv")
    _dev(gate, torch.float32, (B, n, KV), "gate")
    if layer.has_indexer:
        _dev(ikey, torch.float32, (B, n, IDX), "ikey")
        _dev(igate, torch.float32, (B, n, IDX), "igate")
    s = layer.struct()
    _check(lib().lca_compress_append(C.byref(s), _ptr(kv), _ptr(gate), _ptr(ikey), _ptr(igate), n,
                                     _stream()))
    layer.len_min, layer.len_max = s.len_min, s.len_max


def indexer_workspace_bytes(layer: Layer, n_q, H_I, k):
    s = layer.struct()
    return lib().lca_indexer_workspace(C.byref(s), n_q, H_I, k)


def indexer_layout(layer: Layer, n_q, H_I, k):
    """Where the indexer's workspace holds each query's order keys: a dict
    with stride, keys (byte offset), kind (0 full key rows, 1 candidate lists,
    2 per-workgroup candidate segments), zero (bytes at the start that are
    zero between calls) and, for kinds 1 and 2, counts (byte offset), lists
    (lists or segments per query), waves and span."""
    s = layer.struct()
    out = (C.c_int64 * 8)()
    _check(lib().lca_indexer_layout(C.byref(s), n_q, H_I, k, out))
    v = list(out)
    return {"stride": v[0], "keys": v[1], "kind": v[2], "cand": v[2] == 1, "zero": v[3], "counts": v[4],
            "lists": v[5], "waves": v[6], "span": v[7]}


def indexer_topk(layer: Layer, iq, iw, k, out=None):
    """Top-k visible blocks per query.  iq fp32 [B][n_q][H_I][64], iw fp32
    [B][n_q][H_I] -> int32 [B][n_q][k] (ascending, -1 padded)."""
    B, n_q, H_I = iw.shape
    _dev(iq, torch.float32, (B, n_q, H_I, IDX), "iq")
    _dev(iw, torch.float32, (B, n_q, H_I), "iw")
    if out is None:
        out = torch.empty((B, n_q, k), dtype=torch.int32, device=iq.device)
    _dev(out, torch.int32, (B, n_q, k), "topk")
    s = layer.struct()
    nbytes = lib().lca_indexer_workspace(C.byref(s), n_q, H_I, k)
    ws = layer.indexer_workspace(n_q, nbytes)
    _check(lib().lca_indexer_topk(C.byref(s), _ptr(iq), _ptr(iw), n_q, H_I, k, _ptr(out), _ptr(ws),
                                  nbytes, _stream()))
    return out


def decode_append_topk(layer: Layer, kv, gate, ikey, igate, iq, iw, k, out=None):
    """One decode step of a CSA layer up to the top-k (lca_decode_append_topk):
    the same as compress_append(layer, kv, gate, ikey, igate) with one token
    per row followed by indexer_topk(layer, iq, iw, k).  kv [B][1][512]
    bf16 bits, gate [B][1][512], ikey/igate [B][1][64], iq [B][1][H_I][64],
    iw [B][1][H_I] -> int32 [B][1][k]."""
    B = layer.batch
    if kv.dtype == torch.bfloat16:
        kv = kv.view(torch.int16)
    _dev(kv, torch.int16, (B, 1, KV), "kv")
    _dev(gate, torch.float32, (B, 1, KV), "gate")
    _dev(ikey, torch.float32, (B, 1, IDX), "ikey")
    _dev(igate, torch.float32, (B, 1, IDX), "igate")
    H_I = iw.shape[2]
    _dev(iq, torch.float32, (B, 1, H_I, IDX), "iq")
    _dev(iw, torch.float32, (B, 1, H_I), "iw")
    if out is None:
        out = torch.empty((B, 1, k), dtype=torch.int32, device=iq.device)
    _dev(out, torch.int32, (B, 1, k), "topk")
    s = layer.struct()
    nbytes = lib().lca_decode_append_workspace(C.byref(s), H_I, k)
    ws = layer.indexer_workspace(1, nbytes)
    _check(lib().lca_decode_append_topk(C.byref(s), _ptr(kv), _ptr(gate), _ptr(ikey), _ptr(igate), _ptr(iq),
                                        _ptr(iw), H_I, k, _ptr(out), _ptr(ws), nbytes, _stream()))
    layer.len_min, layer.len_max = s.len_min, s.len_max
    return out


def indexer_topk_noalloc(layer: Layer, iq, iw, k, out=None):
    """indexer_topk with the library's static scratch array as workspace
    (lca_indexer_topk_noalloc): no workspace is allocated for the call."""
    B, n_q, H_I = iw.shape
    _dev(iq, torch.float32, (B, n_q, H_I, IDX), "iq")
    _dev(iw, torch.float32, (B, n_q, H_I), "iw")
    if out is None:
        out = torch.empty((B, n_q, k), dtype=torch.int32, device=iq.device)
    _dev(out, torch.int32, (B, n_q, k), "topk")
    s = layer.struct()
    _check(lib().lca_indexer_topk_noalloc(C.byref(s), _ptr(iq), _ptr(iw), n_q, H_I, k, _ptr(out), _stream()))
    return out


def attend_workspace_bytes(layer: Layer, n_q, H, k=0):
    s = layer.struct()
    return lib().lca_attend_workspace(C.byref(s), n_q, H, k)


def _q(q):
    if q.dtype == torch.bfloat16:
        q = q.view(torch.int16)
    return q


def csa_attend(layer: Layer, q, topk, scale=None, out=None):
    """q bf16 [B][n_q][H][512], topk int32 [B][n_q][k] -> fp32 [B][n_q][H][512]."""
    q = _q(q)
    B, n_q, H, _ = q.shape
    k = topk.shape[-1]
    _dev(q, torch.int16, (B, n_q, H, KV), "q")
    _dev(topk, torch.int32, (B, n_q, k), "topk")
    scale = 1.0 / math.sqrt(KV) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, n_q, H, KV), dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, (B, n_q, H, KV), "out")
    s = layer.struct()
    nbytes = lib().lca_attend_workspace(C.byref(s), n_q, H, k)
    ws = layer.workspace(nbytes)
    _check(lib().lca_csa_attend(C.byref(s), _ptr(q), n_q, H, _ptr(topk), k, scale, _ptr(out),
                                _ptr(ws), nbytes, _stream()))
    return out


def hca_attend(layer: Layer, q, scale=None, out=None):
    """q bf16 [B][n_q][H][512] -> fp32 [B][n_q][H][512] over every visible entry + window."""
    q = _q(q)
    B, n_q, H, _ = q.shape
    _dev(q, torch.int16, (B, n_q, H, KV), "q")
    scale = 1.0 / math.sqrt(KV) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, n_q, H, KV), dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, (B, n_q, H, KV), "out")
    s = layer.struct()
    nbytes = lib().lca_attend_workspace(C.byref(s), n_q, H, 0)
    ws = layer.workspace(nbytes)
    _check(lib().lca_hca_attend(C.byref(s), _ptr(q), n_q, H, scale, _ptr(out), _ptr(ws), nbytes,
                                _stream()))
    return out


class KernelTimer:
    """Sum of HIP-event durations of one library kernel over a code region:

        with KernelTimer("indexer_score") as t: ...
        t.total_ms, t.launches, t.durations_ms (one per launch)
    """

    def __init__(self, kernel):
        self.kernel = kernel
        self.total_ms, self.launches = 0.0, 0

    def __enter__(self):
        _check(lib().lca_timing_begin(self.kernel.encode()))
        return self

    def __exit__(self, *exc):
        ms, n = C.c_double(0.0), C.c_int64(0)
        _check(lib().lca_timing_end(C.byref(ms), C.byref(n)))
        self.total_ms, self.launches = ms.value, n.value
        each = (C.c_float * max(1, n.value))()
        _check(lib().lca_timing_durations(each, n.value, C.byref(n)))
        self.durations_ms = [float(x) for x in each[:self.launches]]
        return False
