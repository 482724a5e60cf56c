"""Shared helpers of the GPU parity tests: comparison rules against the oracle.

Tolerances (stated once, used by every GPU test):
  * ring planes, seq_len, indexer scores: bit-exact;
  * top-k index sets: valid (exactly min(k, visible) distinct visible
    blocks, ascending, then -1) and equal to the oracle's, except that a
    block whose oracle score lies within 1e-6 |theta| of theta, the oracle's
    k-th largest score, may be exchanged for another such block (check_topk);
  * compressed entries: the pooled value is fp32 on both sides but the
    device and host exp differ by an ulp now and then, so an FP8/FP4/BF16
    code may differ by one step where the oracle's pre-rounding value lies
    within 1e-5 (relative) of that rounding midpoint; an FP8 scale may differ
    by a few ulps when its amax element does, and an E8M0 exponent by one
    when the amax sits on a power of two (the GPU's codes of that block are
    then checked against the oracle's pooled values under the GPU's
    exponent);
  * attention: per (query, head) row, max|o - o_ref| / max|o_ref| <= 2e-3.
"""
from __future__ import annotations

import numpy as np

import oracle

ATTN_TOL = 2e-3


def e4m3_values():
    return np.array([oracle.e4m3_value(c) for c in range(256)])


_E4 = None


def _e4():
    global _E4
    if _E4 is None:
        _E4 = e4m3_values()
    return _E4


E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _near_mid(t, v1, v2, rel=1e-5):
    mid = (v1 + v2) / 2.0
    return abs(t - mid) <= rel * max(abs(mid), 1e-30)


def compare_entries(gpu, ref_layer, row, blocks, raw_kv, raw_gate, raw_ikey, raw_igate, pos_bias,
                    ipos_bias, m):
    """Compare the GPU's entries of `blocks` with the oracle's pooled-and-
    quantized values, allowing only midpoint flips.  raw_* hold the m tokens
    of each block ([nb][m][C]).  Returns the number of tolerated code flips
    (FP8 scales a few ulps off are checked, not counted)."""
    e4 = _e4()
    flips = 0
    for bi, b in enumerate(blocks):
        x = (raw_kv[bi].astype(np.uint32) << 16).view(np.float32)
        y = oracle.pool(x, raw_gate[bi], pos_bias)
        nope, rope, sc = oracle.make_entry(y)
        g_n, g_r, g_s = gpu["nope"][row, b], gpu["rope"][row, b], gpu["kv_scale"][row, b]
        for g in range(7):
            s_ref, s_gpu = np.float32(sc[g]), np.float32(g_s[g])
            if s_ref != s_gpu:
                # the amax element's pooled value differs by an ulp or so:
                # not a code flip, but a scale a few ulps off
                assert abs(s_ref - s_gpu) <= 4 * np.spacing(s_ref), (row, b, g, s_ref, s_gpu)
            yg = y[g * 64:(g + 1) * 64]
            amax = np.float32(np.abs(yg).max())
            inv = np.float32(448.0) / amax if amax > 0 else np.float32(0)
            for c in range(64):
                cr, cg = nope[g * 64 + c], g_n[g * 64 + c]
                if e4[cr] == e4[cg]:
                    continue
                t = float(np.float32(yg[c]) * inv)
                adjacent = (cr & 0x80) == (cg & 0x80) and abs(int(cr & 0x7F) - int(cg & 0x7F)) == 1
                assert adjacent and _near_mid(t, e4[cr], e4[cg]), (row, b, g, c, t, e4[cr], e4[cg])
                flips += 1
        assert g_s[7] == 0.0
        for c in range(64):
            if rope[c] != g_r[c]:
                # adjacent bf16 codes, the pooled value at their midpoint
                assert abs(int(rope[c]) - int(g_r[c])) == 1, (row, b, c)
                v1 = float((np.array([rope[c]], np.uint32) << 16).view(np.float32)[0])
                v2 = float((np.array([g_r[c]], np.uint32) << 16).view(np.float32)[0])
                assert _near_mid(float(y[448 + c]), v1, v2), (row, b, c, float(y[448 + c]), v1, v2)
                flips += 1
        if ref_layer["has_indexer"]:
            yi = oracle.pool(raw_ikey[bi], raw_igate[bi], ipos_bias)
            code, ex = oracle.make_idx(yi)
            g_c, g_e = gpu["idx_code"][row, b], gpu["idx_scale"][row, b]
            for h in range(2):
                if ex[h] != g_e[h]:
                    # amax sits on a power of two: accept one step of exponent,
                    # then check the codes under the GPU's exponent
                    assert abs(int(ex[h]) - int(g_e[h])) == 1, (row, b, h)
                    amax = float(np.abs(yi[h * 32:(h + 1) * 32]).max())
                    edge = 2.0 ** np.floor(np.log2(amax))
                    assert abs(amax - edge) <= 1e-5 * edge or abs(amax - 2 * edge) <= 1e-5 * edge, (row, b, h)
                    flips += 1
                sc2 = 2.0 ** (int(g_e[h]) - 127)
                for j in range(32):
                    el = h * 32 + j
                    nr = (code[el // 2] >> (4 * (el & 1))) & 15
                    ng = (g_c[el // 2] >> (4 * (el & 1))) & 15
                    if E2M1[nr] == E2M1[ng]:
                        continue
                    t = float(yi[el]) / sc2
                    if ex[h] != g_e[h]:
                        # the oracle's code is for its own exponent: compare
                        # with e2m1 of the value under the GPU's exponent
                        nr = oracle.e2m1_encode(float(np.float32(t)))
                        if E2M1[nr] == E2M1[ng]:
                            continue
                    assert _near_mid(t, E2M1[nr], E2M1[ng]), (row, b, el, t, nr, ng)
                    flips += 1
    return flips


def attn_rel_err(out, ref):
    """max over (query, head) rows of max|o - ref| / max|ref|."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(-1)
    den = np.abs(ref).max(-1)
    return float((num / np.maximum(den, 1e-30)).max())


def decode_keys(keys_u32):
    """order-preserving uint32 keys back to fp32 scores"""
    k = keys_u32.astype(np.uint32)
    bits = np.where(k & 0x80000000, k & 0x7FFFFFFF, ~k).astype(np.uint32)
    return bits.view(np.float32)


def order_keys(scores_f32):
    """fp32 scores to the indexer's uint32 order keys (sign bit set for a
    non-negative score, every bit flipped for a negative one)"""
    u = np.ascontiguousarray(scores_f32, np.float32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def indexer_row_keys(ws, layout, row, nv):
    """(blocks, keys) that the indexer left in its workspace (a uint8 device
    tensor) for query row `row`: every visible block with full key rows, the
    entries of the row's candidate lists otherwise (layout from
    lca.indexer_layout)."""
    import torch
    S = layout["stride"]
    if layout["kind"] == 0:
        k0 = layout["keys"] + row * S * 4
        keys = ws[k0:k0 + S * 4].view(torch.int32).cpu().numpy().view(np.uint32)
        return np.arange(nv), keys[:nv]
    if layout["kind"] == 2:
        # per-workgroup segments of (key, block) pairs: segment s at slot s * span
        k0 = layout["keys"] + row * S * 8
        pairs = ws[k0:k0 + S * 8].view(torch.int32).cpu().numpy().view(np.uint32).reshape(S, 2)
        segs, span = layout["lists"], layout["span"]
        c0 = layout["counts"] + row * segs * 4
        cnt = ws[c0:c0 + segs * 4].view(torch.int32).cpu().numpy().astype(np.int64)
        assert (cnt <= span).all()
        idx = np.concatenate([s_ * span + np.arange(c) for s_, c in enumerate(cnt)]).astype(np.int64) \
            if cnt.sum() else np.zeros(0, np.int64)
        e = pairs[idx]
        blocks = e[:, 1].astype(np.int64)
        # each segment holds blocks of its own range, in ascending order
        seg_of = np.repeat(np.arange(segs), cnt)
        assert ((blocks // span) == seg_of).all()
        return blocks, e[:, 0]
    k0 = layout["keys"] + row * S * 8
    pairs = ws[k0:k0 + S * 8].view(torch.int32).cpu().numpy().view(np.uint32).reshape(S, 2)
    lists, W, span = layout["lists"], layout["waves"], layout["span"]
    c0 = layout["counts"] + row * lists * 4
    cnt = ws[c0:c0 + lists * 4].view(torch.int32).cpu().numpy().astype(np.int64)
    i = np.repeat(np.arange(lists), cnt)                       # list of each entry
    j = np.arange(int(cnt.sum())) - np.repeat(np.cumsum(cnt) - cnt, cnt)   # its index in the list
    g, col = np.divmod(i, 32)
    c, v = np.divmod(g, W)
    assert (c * span + 32 * v + 32 * W * j + col < S).all()
    e = pairs[c * span + 32 * v + 32 * W * j + col]
    return c * span + 32 * (v + W * e[:, 1].astype(np.int64)) + col, e[:, 0]


def check_indexer_keys(blocks, keys, scores, k):
    """The kept keys are the exact order keys of their blocks' oracle scores,
    each block at most once, and every block that can be in the top k is
    kept: all of them when there are at most k, else every block whose key's
    top 12 bits reach those of the k-th largest key."""
    want = order_keys(scores)
    nv = len(want)
    assert len(np.unique(blocks)) == len(blocks), "a block kept twice"
    if len(blocks):
        assert blocks.min() >= 0 and blocks.max() < nv, (blocks.min(), blocks.max(), nv)
    bad = np.nonzero(keys != want[blocks])[0]
    assert bad.size == 0, (blocks[bad[:5]], keys[bad[:5]], want[blocks[bad[:5]]])
    if nv <= k:
        need = np.arange(nv)
    else:
        tb = np.sort(want)[nv - k] >> 20
        need = np.nonzero((want >> 20) >= tb)[0]
    missing = np.setdiff1d(need, blocks)
    assert missing.size == 0, ("blocks that can reach the top k are missing", missing[:5])


TOPK_REL = 1e-6


def check_topk(got, want, scores, k, rel=TOPK_REL):
    """One query's selection against the oracle's.  got / want: the k output
    slots; scores: the oracle's score of every visible block.  The output
    holds exactly min(k, visible) distinct visible blocks in ascending order,
    then -1; every block in the symmetric difference with the oracle's set
    has an oracle score within rel * |theta| of theta, the oracle's k-th
    largest score.  Returns True when the two sets are equal."""
    got = np.asarray(got, np.int64)
    want = np.asarray(want, np.int64)
    scores = np.asarray(scores, np.float32)
    nv = len(scores)
    n = min(k, nv)
    assert got.shape == (k,) and want.shape == (k,)
    assert np.all(got[n:] == -1), "slots past min(k, visible) must be -1"
    sel = got[:n]
    assert np.all((sel >= 0) & (sel < nv)), "an output block is not visible"
    assert np.all(np.diff(sel) > 0), "output blocks must be distinct and ascending"
    if np.array_equal(got, want):
        return True
    theta = np.sort(scores.astype(np.float64))[::-1][n - 1]
    diff = np.setxor1d(sel, want[:n])
    off = np.abs(scores[diff].astype(np.float64) - theta) > rel * abs(theta)
    assert not off.any(), ("blocks outside the tie band differ", diff[off][:5], scores[diff[off][:5]], theta)
    return False
