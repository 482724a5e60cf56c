"""Seeded cache images, raw token streams and queries for the workloads.

Everything here is random data laid out in the cache's plane layout; no step
of the method (pooling, quantization, scoring, attention) is performed.
Cache images are random codes:
  * nope: random e4m3fn bytes (NaN codes moved to +-448), per-64 fp32 scales
    uniform in [2/448, 3/448], slot 7 of each scale row 0;
  * rope: bf16 of N(0,1);
  * indexer keys: random e2m1 nibbles with E8M0 block exponents 2^-3..2^0;
  * ring: the last min(len, R) raw tokens (bf16 N(0,1) KV, N(0,1) gates and
    indexer streams) at slot position % R.
Needle blocks (retrieval stand-ins) get indexer codes equal to the sign
pattern of sum_h w_h q_h at the largest e2m1 magnitude with block exponent
2^1, and KV codes with the sign pattern of sum_h q_h at a large e4m3
magnitude, so that they outrank random blocks for the query they target.
Every tensor comes from its own stream (seed, name, row), so one row can be
regenerated alone.
"""
from __future__ import annotations

import numpy as np

from . import (bf16_bits, bf16_to_f32, abs_normal_f32, bf16_normal, distinct_choice, e2m1_code_image,
               e4m3_code_image, e8m0_image, fp8_scale_image, key, normal_f32, randbytes, u64)

KV, NOPE, ROPE, IDX = 512, 448, 64, 64


def empty_layer(batch, ratio, window, ring, has_indexer, max_blocks):
    B, MB, R = batch, max_blocks, ring
    L = dict(batch=B, ratio=ratio, window=window, ring=R, has_indexer=int(has_indexer),
             max_blocks=MB,
             seq_len=np.zeros(B, np.int32),
             nope=np.zeros((B, MB, NOPE), np.uint8),
             rope=np.zeros((B, MB, ROPE), np.uint16),
             kv_scale=np.zeros((B, MB, 8), np.float32),
             idx_code=np.zeros((B, MB if has_indexer else 0, 32), np.uint8),
             idx_scale=np.zeros((B, MB if has_indexer else 0, 2), np.uint8),
             ring_kv=np.zeros((B, R, KV), np.uint16),
             ring_gate=np.zeros((B, R, KV), np.float32),
             ring_ikey=np.zeros((B, R if has_indexer else 0, IDX), np.float32),
             ring_igate=np.zeros((B, R if has_indexer else 0, IDX), np.float32))
    return L


def pos_bias(seed, tag, ratio, has_indexer):
    pb = normal_f32(seed, "pos_bias", (ratio, KV), tag)
    ipb = normal_f32(seed, "ipos_bias", (ratio, IDX), tag) if has_indexer else None
    return pb, ipb


def fill_row_image(L, seed, tag, row, length):
    """Random cache image for row `row` holding `length` tokens."""
    m, R, MB = L["ratio"], L["ring"], L["max_blocks"]
    nb = length // m
    if nb > MB:
        raise ValueError("cache capacity exceeded")
    L["seq_len"][row] = length
    if nb:
        L["nope"][row, :nb] = e4m3_code_image(seed, "nope", nb * NOPE, tag, row).reshape(nb, NOPE)
        L["rope"][row, :nb] = bf16_normal(seed, "rope", (nb, ROPE), tag, row)
        sc = fp8_scale_image(seed, "kv_scale", nb * 7, tag, row).reshape(nb, 7)
        L["kv_scale"][row, :nb, :7] = sc
        L["kv_scale"][row, :nb, 7] = 0.0
        if L["has_indexer"]:
            L["idx_code"][row, :nb] = e2m1_code_image(seed, "idx_code", nb * 32, tag, row).reshape(nb, 32)
            L["idx_scale"][row, :nb] = e8m0_image(seed, "idx_scale", nb * 2, tag, row).reshape(nb, 2)
    nr = min(length, R)
    if nr:
        pos = np.arange(length - nr, length)
        slots = pos % R
        L["ring_kv"][row, slots] = bf16_normal(seed, "ring_kv", (nr, KV), tag, row)
        L["ring_gate"][row, slots] = normal_f32(seed, "ring_gate", (nr, KV), tag, row)
        if L["has_indexer"]:
            L["ring_ikey"][row, slots] = normal_f32(seed, "ring_ikey", (nr, IDX), tag, row)
            L["ring_igate"][row, slots] = normal_f32(seed, "ring_igate", (nr, IDX), tag, row)


def make_layer(seed, tag, batch, ratio, window, ring, has_indexer, max_blocks, lengths):
    L = empty_layer(batch, ratio, window, ring, has_indexer, max_blocks)
    L["pos_bias"], L["ipos_bias"] = pos_bias(seed, tag, ratio, has_indexer)
    for b in range(batch):
        fill_row_image(L, seed, tag, b, int(lengths[b]))
    return L


def tokens(seed, tag, batch, n, has_indexer, step=0):
    """Raw tokens for one append of n tokens per row."""
    t = dict(kv=bf16_normal(seed, "tok_kv", (batch, n, KV), tag, step),
             gate=normal_f32(seed, "tok_gate", (batch, n, KV), tag, step))
    if has_indexer:
        t["ikey"] = normal_f32(seed, "tok_ikey", (batch, n, IDX), tag, step)
        t["igate"] = normal_f32(seed, "tok_igate", (batch, n, IDX), tag, step)
    return t


def queries(seed, tag, batch, n_q, H, H_I=0, step=0):
    q = dict(q=bf16_normal(seed, "q", (batch, n_q, H, KV), tag, step))
    if H_I:
        q["iq"] = normal_f32(seed, "iq", (batch, n_q, H_I, IDX), tag, step)
        q["iw"] = abs_normal_f32(seed, "iw", (batch, n_q, H_I), tag, step)
    return q


def signed_weights(seed, tag, iw, mode):
    """Indexer weights of another sign pattern, from |N(0,1)| weights iw:
    "abs" leaves them, "neg" negates them all, "mixed" flips a seeded random
    half of them."""
    if mode == "abs":
        return iw
    if mode == "neg":
        return (-iw).astype(np.float32)
    flip = (randbytes(key(seed, "iw_sign", tag), iw.size) & 1).reshape(iw.shape).astype(bool)
    return np.where(flip, -iw, iw).astype(np.float32)


def plant_needles(L, seed, tag, row, count, iq_row, iw_row, q_row):
    """Plant `count` needle blocks in `row`, targeted at one query (its fp32
    indexer query [H_I][64], weights [H_I] and bf16-bit attention query
    [H][512]).  Returns the needle block indices.  Needles lie outside the
    query's window: blocks 0 .. n_vis - 1 - ceil(W/m)."""
    m, W = L["ratio"], L["window"]
    n_vis = int(L["seq_len"][row]) // m
    hi = n_vis - 1 - (W + m - 1) // m
    blocks = distinct_choice(seed, "needles", count, 0, hi, tag, row)
    u = (iw_row[:, None].astype(np.float64) * iq_row.astype(np.float64)).sum(0)
    nib = np.where(u < 0, 0xF, 0x7).astype(np.uint8)          # +-6
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    qsum = (q_row.astype(np.uint32) << 16).view(np.float32).astype(np.float64).sum(0)
    kv_code = np.where(qsum[:NOPE] < 0, 0xEE, 0x6E).astype(np.uint8)  # +-112
    for b in blocks:
        L["idx_code"][row, b] = packed
        L["idx_scale"][row, b] = 128
        L["nope"][row, b] = kv_code
    return blocks


def outlier_channels(seed, tag, layer, count=26):
    """`count` distinct KV channels (of 512) that carry outliers in one layer."""
    return np.sort(distinct_choice(seed, "outliers", count, 0, KV - 1, tag, layer)).astype(np.int64)


def apply_outliers(L, ch, factor=20.0):
    """Stress pattern on a cache image: every FP8 group holding an outlier
    channel gets its scale multiplied by `factor`, outlier RoPE dims and the
    ring's raw tokens in those channels are multiplied by `factor` (bf16)."""
    groups = np.unique(ch[ch < NOPE] // 64)
    for g in groups:
        L["kv_scale"][:, :, g] *= np.float32(factor)
    rc = ch[ch >= NOPE] - NOPE
    if rc.size:
        L["rope"][:, :, rc] = bf16_bits(bf16_to_f32(L["rope"][:, :, rc]) * np.float32(factor))
    L["ring_kv"][:, :, ch] = bf16_bits(bf16_to_f32(L["ring_kv"][:, :, ch]) * np.float32(factor))


def outlier_tokens(tok, ch, factor=20.0):
    """The same stress on a batch of raw tokens (in place)."""
    tok["kv"][:, :, ch] = bf16_bits(bf16_to_f32(tok["kv"][:, :, ch]) * np.float32(factor))
    return tok


ENTRY_PLANES = ("nope", "rope", "kv_scale", "idx_code", "idx_scale")


def paginate(L, seed, page_blocks, reserve_blocks=0, spare_pages=3):
    """The same layer with paged entry planes: each row maps the pages its
    entries need (its current blocks plus `reserve_blocks` more, up to
    max_blocks), every row's pages drawn from one pool in a seeded random
    order; the remaining logical pages are unmapped (-1).  `spare_pages`
    extra pool pages hold random codes that no row maps (a wrong page read
    shows up).  Entry planes become [pool_pages * page_blocks][...]; the
    other planes are copies."""
    PB, B, MB, m = int(page_blocks), L["batch"], L["max_blocks"], L["ratio"]
    assert MB % PB == 0
    ppr = MB // PB
    need = [min(ppr, (int(L["seq_len"][r]) // m + reserve_blocks + PB - 1) // PB) for r in range(B)]
    pool = sum(need) + spare_pages
    order = np.argsort(u64(key(seed, "page_order", B, PB), pool), kind="stable").astype(np.int32)
    P = dict(L)
    for f in ("seq_len", "ring_kv", "ring_gate", "ring_ikey", "ring_igate"):
        P[f] = L[f].copy()                       # appends mutate these in place
    P["page_blocks"], P["pool_pages"] = PB, pool
    table = np.full((B, ppr), -1, np.int32)
    E = pool * PB
    has_idx = bool(L["has_indexer"])
    P["nope"] = e4m3_code_image(seed, "pool_nope", E * NOPE, PB).reshape(E, NOPE)
    P["rope"] = bf16_normal(seed, "pool_rope", (E, ROPE), PB)
    sc = np.zeros((E, 8), np.float32)
    sc[:, :7] = fp8_scale_image(seed, "pool_scale", E * 7, PB).reshape(E, 7)
    P["kv_scale"] = sc
    if has_idx:
        P["idx_code"] = e2m1_code_image(seed, "pool_idx", E * 32, PB).reshape(E, 32)
        P["idx_scale"] = e8m0_image(seed, "pool_iscale", E * 2, PB).reshape(E, 2)
    else:
        P["idx_code"] = np.zeros((0, 32), np.uint8)
        P["idx_scale"] = np.zeros((0, 2), np.uint8)
    nxt = 0
    for r in range(B):
        for j in range(need[r]):
            pg = int(order[nxt])
            nxt += 1
            table[r, j] = pg
            src = slice(j * PB, (j + 1) * PB)
            dst = slice(pg * PB, (pg + 1) * PB)
            for f in ENTRY_PLANES:
                if f.startswith("idx") and not has_idx:
                    continue
                P[f][dst] = L[f][r, src]
    P["page_table"] = table
    return P


def unpaginate(P):
    """The contiguous layer holding a paged layer's mapped entries (unmapped
    pages read as zeros)."""
    B, MB, PB = P["batch"], P["max_blocks"], P["page_blocks"]
    L = dict(P)
    for k in ("page_blocks", "pool_pages", "page_table"):
        L.pop(k)
    for f in ENTRY_PLANES:
        src = P.get(f)
        if src is None:
            continue
        if src.shape[0] == 0:
            L[f] = np.zeros((B, 0) + src.shape[1:], src.dtype)
            continue
        out = np.zeros((B, MB) + src.shape[1:], src.dtype)
        for r in range(B):
            for j, pg in enumerate(P["page_table"][r]):
                if pg >= 0:
                    out[r, j * PB:(j + 1) * PB] = src[pg * PB:(pg + 1) * PB]
        L[f] = out
    return L
