"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every case prints its name, shape and seed before touching the GPU.  Inputs
come from synth (seeded); expected values come from the oracle only.
"""
import os
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from synth import layers as SL

from gpu_helpers import (ATTN_TOL, attn_rel_err, check_indexer_keys, check_topk, compare_entries,
                         indexer_row_keys)

pytestmark = pytest.mark.gpu
SCALE = np.float32(1.0 / np.sqrt(512.0))


def _lca():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_append_amd as lca
    return lca


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


# ------------------------------------------------------------------ compressor

COMPRESS_CASES = [
    # (name, ratio, has_idx, window, ring, batch, initial lengths, append sizes)
    ("csa_m4", 4, 1, 16, 64, 3, [0, 5, 11], [37, 1, 1, 1, 1, 9, 3]),
    ("hca_m128", 128, 0, 16, 300, 2, [0, 100], [130, 1, 1, 60, 70]),
    ("m1_idx", 1, 1, 8, 40, 2, [0, 3], [20, 1, 7]),
    ("m8_noidx", 8, 0, 32, 96, 1, [0], [57, 1, 1, 1, 30]),
    # every ratio of the supported range: 2 (registers), 16 (LDS batches of
    # 16 tokens), 32 and 64 (batches of 32), with and without the indexer
    ("m2_idx", 2, 1, 4, 32, 2, [0, 1], [9, 1, 1, 5]),
    ("m16_idx", 16, 1, 16, 64, 2, [0, 7], [40, 1, 1, 30, 9]),
    ("m16_noidx", 16, 0, 16, 64, 1, [5], [27, 16, 1]),
    ("m32_noidx", 32, 0, 16, 128, 2, [0, 20], [70, 1, 33, 1]),
    ("m64_idx", 64, 1, 8, 200, 1, [0], [130, 1, 63, 2]),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=[c[0] for c in COMPRESS_CASES])
def test_compress_append_parity(case):
    lca = _lca()
    name, m, hi, W, R, B, lens0, appends = case
    seed = 2000 + zlib.crc32(name.encode()) % 1000
    say("compress", name, "m", m, "idx", hi, "B", B, "appends", appends, "seed", seed)
    total = max(lens0) + sum(appends)
    MB = total // m + 2
    # history of raw tokens per row (positions 0..total-1)
    hist = SL.tokens(seed, "hist", B, total, hi)
    ref = SL.empty_layer(B, m, W, R, hi, MB)
    ref["pos_bias"], ref["ipos_bias"] = SL.pos_bias(seed, name, m, hi)
    # initial state: row b holds lens0[b] tokens, appended on the oracle side
    # token by token (rows with fewer tokens get theirs first)
    for b in range(B):
        one = SL.empty_layer(1, m, W, R, hi, MB)
        one["pos_bias"], one["ipos_bias"] = ref["pos_bias"], ref["ipos_bias"]
        if lens0[b]:
            oracle.compress_append(one, hist["kv"][b:b + 1, :lens0[b]].copy(),
                                   hist["gate"][b:b + 1, :lens0[b]].copy(),
                                   hist["ikey"][b:b + 1, :lens0[b]].copy() if hi else None,
                                   hist["igate"][b:b + 1, :lens0[b]].copy() if hi else None)
        for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
                  "ring_gate", "ring_ikey", "ring_igate"):
            ref[f][b] = one[f][0]
    lay = lca.Layer.from_host(ref)
    pos = np.array(lens0)
    for n in appends:
        idx = pos[:, None] + np.arange(n)[None, :]
        rows = np.arange(B)[:, None]
        tk = {k: np.ascontiguousarray(v[rows, idx]) for k, v in hist.items()}
        oracle.compress_append(ref, tk["kv"], tk["gate"], tk.get("ikey"), tk.get("igate"))
        lca.compress_append(lay, _dev(tk["kv"]), _dev(tk["gate"]),
                            _dev(tk["ikey"]) if hi else None, _dev(tk["igate"]) if hi else None)
        pos = pos + n
    torch.cuda.synchronize()
    got = lay.download()
    assert np.array_equal(got["seq_len"], ref["seq_len"])
    assert lay.len_min == pos.min() and lay.len_max == pos.max()
    for f in ("ring_kv", "ring_gate", "ring_ikey", "ring_igate"):
        if ref[f].size:
            assert np.array_equal(got[f], ref[f]), f
    flips = 0
    for b in range(B):
        nb = int(pos[b]) // m
        blocks = list(range(nb))
        t = np.arange(nb * m).reshape(nb, m)
        flips += compare_entries(got, ref, b, blocks, hist["kv"][b][t], hist["gate"][b][t],
                                 hist["ikey"][b][t] if hi else None,
                                 hist["igate"][b][t] if hi else None, ref["pos_bias"],
                                 ref["ipos_bias"], m)
        assert not got["nope"][b, nb:].any()
    n_codes = sum(int(p) // m for p in pos) * (448 + 64 + (64 if hi else 0))
    assert flips <= max(2, n_codes // 1000), flips


# ------------------------------------------------------------------ indexer

INDEXER_CASES = [
    # (name, batch, lengths, n_q, H_I, k, needles)
    ("tiny_h4_k64", 1, [4096], 1, 4, 64, 4),
    ("ragged_h16_k512", 3, [9000, 4100, 6001], 1, 16, 512, 16),
    ("prefill_nq5_h16", 2, [3000, 2999], 5, 16, 128, 0),
    ("h20_two_groups", 2, [2500, 2600], 2, 20, 100, 0),
    ("h32_k2048", 1, [12000], 1, 32, 2048, 0),
    ("k_ge_visible", 2, [200, 37], 1, 8, 64, 0),
    # more than one selection round of 32768 blocks
    ("long_rows_h16_k512", 2, [140000, 70000], 1, 16, 512, 16),
    ("long_nq2_h8_k256", 1, [200000], 2, 8, 256, 0),
    # many queries per row (prefill chunks)
    ("chunk_nq64_h16_k256", 2, [30000, 20011], 64, 16, 256, 0),
    ("chunk_nq37_h32_k128", 1, [9000], 37, 32, 128, 0),
    ("chunk_nq20_h5_k64", 2, [3000, 2100], 20, 5, 64, 0),
    # a chunk right after a short prior: the first queries see at most k
    # blocks, the later ones a few more
    ("chunk_short_prior_k64", 1, [300], 64, 16, 64, 0),
    # the smallest shapes: one indexer head, k = 1
    ("h1_k1", 2, [4000, 2001], 1, 1, 1, 0),
    ("chunk_nq16_h1_k1", 1, [3000], 16, 1, 1, 0),
    # weights of either sign: negative scores, and with all weights negative
    # every block whose dots are all <= 0 ties at +0 (ranked by index)
    ("negw_h16_k128", 2, [9000, 5000], 1, 16, 128, 0, "neg"),
    ("mixw_h16_k512", 2, [30000, 11000], 1, 16, 512, 0, "mixed"),
    ("mixw_h4_k64", 1, [4096], 1, 4, 64, 0, "mixed"),
    ("mixw_h32_nq3_k300", 1, [12000], 3, 32, 300, 0, "mixed"),
    ("mixw_chunk_nq40_h16_k256", 1, [20000], 40, 16, 256, 0, "mixed"),
    ("negw_chunk_nq24_h24_k64", 1, [9000], 24, 24, 64, 0, "neg"),
    ("mixw_long_h8_k256", 1, [140000], 1, 8, 256, 0, "mixed"),
]

# environment switches: the selection split over workgroups, the score
# kernel that shares key tiles across a row's queries, with candidate lists
# where a row has at most 64 of them (tile), always (tile_cand) or never
# (tile_full); with fused, one query per row selects inside the scoring
# launch
INDEXER_MODES = {"auto": {}, "sliced": {"LCA_TOPK_SLICED": "1"}, "tile": {"LCA_SCORE_TILE": "1"},
                 "tile_cand": {"LCA_SCORE_TILE": "1", "LCA_TOPK_CAND": "1"},
                 "tile_full": {"LCA_SCORE_TILE": "1", "LCA_TOPK_CAND": "0"},
                 "no_tile": {"LCA_SCORE_TILE": "0"},
                 "separate": {"LCA_TOPK_FUSED": "0", "LCA_TOPK_SLICED": "0"}}

# oracle results per case, shared by the modes
_ORACLE = {}


def _indexer_case(lca, name, B, lens, n_q, H_I, k, needles, seed, wsign="abs"):
    m, W = 4, 128
    MB = max(lens) // m + 8
    ref = SL.make_layer(seed, name, B, m, W, 256, 1, MB, lens)
    Q = SL.queries(seed, name, B, n_q, 16, H_I)
    Q["iw"] = SL.signed_weights(seed, name, Q["iw"], wsign)
    if needles:
        for b in range(B):
            SL.plant_needles(ref, seed, name, b, needles, Q["iq"][b, -1], Q["iw"][b, -1],
                             Q["q"][b, -1])
    lay = lca.Layer.from_host(ref)
    return ref, lay, Q


@pytest.mark.parametrize("mode", list(INDEXER_MODES))
@pytest.mark.parametrize("case", INDEXER_CASES, ids=[c[0] for c in INDEXER_CASES])
def test_indexer_topk_parity(case, mode, tuning):
    lca = _lca()
    name, B, lens, n_q, H_I, k, needles = case[:7]
    wsign = case[7] if len(case) > 7 else "abs"
    seed = 3000 + len(name)
    say("indexer", name, "B", B, "lens", lens, "n_q", n_q, "H_I", H_I, "k", k, "seed", seed, "mode", mode,
        "weights", wsign)
    for var, val in INDEXER_MODES[mode].items():
        tuning(var, val)
    ref, lay, Q = _indexer_case(lca, name, B, lens, n_q, H_I, k, needles, seed, wsign)
    got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    if name not in _ORACLE:
        _ORACLE[name] = (oracle.indexer_topk(ref, Q["iq"], Q["iw"], k),
                         [[oracle.indexer_scores(ref, b, qi, n_q, Q["iq"], Q["iw"]) for qi in range(n_q)]
                          for b in range(B)])
    want, scores = _ORACLE[name]
    # scores: the workspace holds the order keys of every visible block, or
    # of every block that can reach the top k (candidate lists)
    ws = lay.indexer_workspace(n_q)
    layout = lca.indexer_layout(lay, n_q, H_I, k)
    assert layout["zero"] >= B * n_q * 4096 * 4
    assert not ws[:layout["zero"]].view(torch.int32).any().item()   # counters, histograms zeroed for the next call
    for b in range(B):
        for qi in range(n_q):
            sc = scores[b][qi]
            blocks, keys = indexer_row_keys(ws, layout, b * n_q + qi, len(sc))
            check_indexer_keys(blocks, keys, sc, k)
            check_topk(got[b, qi], want[b, qi], sc, k)
    if needles:
        for b in range(B):
            nd = SL.plant_needles(ref, seed, name, b, needles, Q["iq"][b, -1], Q["iw"][b, -1],
                                  Q["q"][b, -1])
            assert set(nd) <= set(got[b, -1].tolist())
    assert lay.status() == 0


def test_indexer_prefill_decode_prefill_one_layer():
    """One layer serves a prefill chunk (64 queries per row), then a decode
    step (1 query per row), then another chunk: each call's selection
    matches the oracle.  The decode call's data must not land where the
    chunk's histograms lie (each query count has a workspace of its own)."""
    lca = _lca()
    B, L, H_I, k = 2, 30000, 16, 256
    say("indexer prefill, decode, prefill on one layer", B, L)
    ref = SL.make_layer(93, "pdp", B, 4, 128, 256, 1, L // 4 + 8, [L, L - 9])
    lay = lca.Layer.from_host(ref)
    for step, n_q in enumerate((64, 1, 64)):
        Q = SL.queries(93, "pdp", B, n_q, 16, H_I, step=step)
        got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k).cpu().numpy()
        want = oracle.indexer_topk(ref, Q["iq"], Q["iw"], k)
        for b in range(B):
            for qi in (0, n_q // 2, n_q - 1):
                check_topk(got[b, qi], want[b, qi], oracle.indexer_scores(ref, b, qi, n_q, Q["iq"], Q["iw"]), k)


TIE_MODES = ["auto", "sliced", "tile_cand", "separate"]


@pytest.mark.parametrize("mode", TIE_MODES)
@pytest.mark.parametrize("B,L", [(1, 4000), (2, 140000)], ids=["short", "long"])
def test_indexer_equal_scores_take_lowest_indices(B, L, mode, tuning):
    lca = _lca()
    say("indexer equal scores", B, L, "mode", mode)
    for var, val in INDEXER_MODES[mode].items():
        tuning(var, val)
    m, k = 4, 50
    ref = SL.make_layer(77, "eq", B, m, 128, 256, 1, L // m + 4, [L] * B)
    ref["idx_code"][:] = 0x22          # every key identical
    ref["idx_scale"][:] = 127
    Q = SL.queries(77, "eq", B, 1, 16, 4)
    lay = lca.Layer.from_host(ref)
    got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k).cpu().numpy()
    want = oracle.indexer_topk(ref, Q["iq"], Q["iw"], k)
    assert np.array_equal(got, want)
    for b in range(B):
        assert list(got[b, 0]) == list(range(k))


@pytest.mark.parametrize("mode", TIE_MODES)
@pytest.mark.parametrize("L", [48000, 140000], ids=["one_round", "two_rounds"])
def test_indexer_near_equal_scores(L, mode, tuning):
    """Most scores share their high bits (keys differ in one byte): exercises
    the second-level candidate selection."""
    lca = _lca()
    say("indexer near-equal scores", L, "mode", mode)
    for var, val in INDEXER_MODES[mode].items():
        tuning(var, val)
    B, m, k = 2, 4, 512
    ref = SL.make_layer(78, "neq", B, m, 128, 256, 1, L // m + 4, [L, L - 7])
    rng = np.random.default_rng(78)
    pattern = rng.integers(0, 256, 32).astype(np.uint8)
    ref["idx_code"][:] = pattern
    ref["idx_code"][:, :, 5] = rng.integers(0, 256, ref["idx_code"].shape[:2]).astype(np.uint8)
    ref["idx_scale"][:] = 126
    Q = SL.queries(78, "neq", B, 1, 16, 16)
    lay = lca.Layer.from_host(ref)
    got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k).cpu().numpy()
    want = oracle.indexer_topk(ref, Q["iq"], Q["iw"], k)
    for b in range(B):
        check_topk(got[b, 0], want[b, 0], oracle.indexer_scores(ref, b, 0, 1, Q["iq"], Q["iw"]), k)


@pytest.mark.parametrize("mode", ["tile", "tile_full", "no_tile"])
def test_indexer_exponent_extremes(mode, tuning):
    """Key halves with E8M0 scales up to 12 apart and query halves scaled by
    2^20 or 2^-12: the products of the two MX halves can no longer be added
    inside one matrix-core product without rounding, so the per-half path
    runs.  (Exponent gaps stay below ~35 so that the oracle's double sum of
    the two halves is itself exact.)"""
    lca = _lca()
    say("indexer exponent extremes", mode)
    for var, val in INDEXER_MODES[mode].items():
        tuning(var, val)
    B, m, L, n_q, H_I, k = 2, 4, 6000, 24, 16, 100
    ref = SL.make_layer(79, "ext", B, m, 128, 256, 1, L // m + 4, [L, L - 3])
    rng = np.random.default_rng(79)
    sc = ref["idx_scale"]
    sel = rng.random(sc.shape[:2]) < 0.3
    sc[sel, 0] = np.clip(sc[sel, 0].astype(np.int32) + rng.integers(-12, 13, sel.sum()), 1, 254).astype(np.uint8)
    Q = SL.queries(79, "ext", B, n_q, 16, H_I)
    iq = Q["iq"].copy()
    iq[:, :8, :, :32] *= np.float32(2.0 ** 20)      # the first query group: per-half path throughout
    iq[:, 9::3, 3, 32:] *= np.float32(2.0 ** -12)
    lay = lca.Layer.from_host(ref)
    got = lca.indexer_topk(lay, _dev(iq), _dev(Q["iw"]), k).cpu().numpy()
    want = oracle.indexer_topk(ref, iq, Q["iw"], k)
    for b in range(B):
        for qi in range(n_q):
            check_topk(got[b, qi], want[b, qi], oracle.indexer_scores(ref, b, qi, n_q, iq, Q["iw"]), k)


_MAX_CASE = {}


@pytest.mark.parametrize("mode", ["auto", "single", "sliced"])
def test_indexer_max_blocks(mode, tuning):
    """The longest row the indexer takes: 524 288 blocks (2^21 tokens at
    m = 4), which fills the whole selection bitmap: the selection inside the
    scoring launch (the default: 256 candidate segments), 16 rounds of the
    single selection workgroup, or 32 part workgroups of the sliced one."""
    lca = _lca()
    say("indexer max blocks", mode)
    env = {"auto": {}, "single": {"LCA_TOPK_SLICED": "0", "LCA_TOPK_FUSED": "0"},
           "sliced": {"LCA_TOPK_SLICED": "1"}}[mode]
    for var, val in env.items():
        tuning(var, val)
    B, m, k, H_I, MB = 1, 4, 256, 8, 524288
    if not _MAX_CASE:
        ref = SL.make_layer(80, "max", B, m, 128, 256, 1, MB, [MB * m])
        Q = SL.queries(80, "max", B, 1, 16, H_I)
        _MAX_CASE.update(ref=ref, Q=Q, want=oracle.indexer_topk(ref, Q["iq"], Q["iw"], k),
                         scores=oracle.indexer_scores(ref, 0, 0, 1, Q["iq"], Q["iw"]))
    ref, Q, want = _MAX_CASE["ref"], _MAX_CASE["Q"], _MAX_CASE["want"]
    lay = lca.Layer.from_host(ref)
    got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k).cpu().numpy()
    check_topk(got[0, 0], want[0, 0], _MAX_CASE["scores"], k)


# ------------------------------------------------------------------ attention

ATTEND_CASES = [
    # (name, csa, batch, lengths, n_q, H, k, splits)
    ("hca_h16_small", 0, 1, [4096], 1, 16, 0, 0),
    ("hca_h64_ragged", 0, 3, [20000, 9001, 300], 1, 64, 0, 0),
    ("hca_h64_onesplit", 0, 2, [3000, 2000], 1, 64, 0, 1),
    ("hca_nq4_h20", 0, 2, [5000, 4000], 4, 20, 0, 3),
    ("csa_h64_k512", 1, 2, [9000, 6000], 1, 64, 512, 0),
    ("csa_h16_k64_pad", 1, 2, [300, 100], 2, 16, 64, 0),
    ("csa_h64_k512_onesplit", 1, 1, [8000], 1, 64, 512, 1),
    ("short_rows", 0, 2, [1, 3], 1, 64, 0, 0),
    # the largest shapes the ABI takes: 128 heads (two head groups), k = 2048
    # (more keys than one split stages)
    ("csa_h128_k2048", 1, 1, [12000], 2, 128, 2048, 0),
    ("hca_h128_onesplit", 0, 1, [40000], 1, 128, 0, 1),
    # many query rows of one chunk each (more workgroups than CUs), rows
    # with a short window among them
    ("csa_rows_nq300_h64_k64", 1, 2, [3000, 400], 300, 64, 64, 0),
    ("csa_rows_nq200_h128_k96", 1, 1, [5000], 200, 128, 96, 0),
]


@pytest.mark.parametrize("case", ATTEND_CASES, ids=[c[0] for c in ATTEND_CASES])
def test_attend_parity(case, tuning):
    lca = _lca()
    name, csa, B, lens, n_q, H, k, splits = case
    seed = 4000 + len(name) * 7 + csa
    say("attend", name, "csa", csa, "B", B, "lens", lens, "n_q", n_q, "H", H, "k", k,
        "splits", splits, "seed", seed)
    if splits:
        tuning("LCA_ATTEND_SPLITS", splits)
    m = 4 if csa else 128
    W = 128
    MB = max(lens) // m + 8
    R = max(256, n_q + W)
    ref = SL.make_layer(seed, name, B, m, W, R, csa, MB, lens)
    Q = SL.queries(seed, name, B, n_q, H)
    lay = lca.Layer.from_host(ref)
    q = _dev(Q["q"])
    if csa:
        # a selection list with padding, invisible entries and unsorted order
        rng = np.random.default_rng(seed)
        topk = np.full((B, n_q, k), -1, np.int32)
        for b in range(B):
            for qi in range(n_q):
                p = lens[b] - n_q + qi
                nv = (p + 1) // m
                take = min(k - 2, nv)
                sel = rng.choice(nv, size=take, replace=False) if nv else np.zeros(0, int)
                topk[b, qi, :take] = np.sort(sel)
                if take < k:
                    topk[b, qi, take] = nv + 3          # not visible: ignored
        want = oracle.csa_attend(ref, Q["q"], topk, SCALE)
        got = lca.csa_attend(lay, q, _dev(topk), float(SCALE))
    else:
        want = oracle.hca_attend(ref, Q["q"], SCALE)
        got = lca.hca_attend(lay, q, float(SCALE))
    torch.cuda.synchronize()
    err = attn_rel_err(got.cpu().numpy(), want)
    print("max rel err", err)
    assert err <= ATTN_TOL
    assert lay.status() == 0
    # the same call twice gives bitwise-identical output (no races in LDS)
    again = (lca.csa_attend(lay, q, _dev(topk), float(SCALE)) if csa
             else lca.hca_attend(lay, q, float(SCALE)))
    torch.cuda.synchronize()
    assert torch.equal(again, got)


def test_attend_outlier_channels():
    """FP8 scales stressed by x20 outlier channels (5% of KV channels)."""
    lca = _lca()
    say("attend outliers")
    seed, B, lens, H, m = 5150, 2, [30000, 20000], 64, 128
    ref = SL.make_layer(seed, "out", B, m, 128, 256, 0, max(lens) // m + 4, lens)
    rng = np.random.default_rng(seed)
    ch = rng.choice(512, 26, replace=False)
    big = ch[ch < 448]
    # every FP8 group holding an outlier channel gets a x20 scale (once)
    for g in np.unique(big // 64):
        ref["kv_scale"][:, :, g] *= 20.0
    rope_ch = ch[ch >= 448] - 448
    vals = synth.bf16_to_f32(ref["rope"][:, :, rope_ch]) * 20.0
    ref["rope"][:, :, rope_ch] = synth.bf16_bits(vals)
    rk = synth.bf16_to_f32(ref["ring_kv"][:, :, ch]) * 20.0
    ref["ring_kv"][:, :, ch] = synth.bf16_bits(rk)
    Q = SL.queries(seed, "out", B, 1, H)
    lay = lca.Layer.from_host(ref)
    got = lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
    want = oracle.hca_attend(ref, Q["q"], SCALE)
    err = attn_rel_err(got.cpu().numpy(), want)
    print("max rel err", err)
    assert err <= ATTN_TOL


# ------------------------------------------------------------------ errors

def test_errors_enqueue_nothing():
    lca = _lca()
    say("errors")
    lay = lca.Layer(1, 4, 16, 32, True, 16)
    kv = torch.zeros((1, 40, 512), dtype=torch.int16, device="cuda")
    g = torch.zeros((1, 40, 512), dtype=torch.float32, device="cuda")
    ik = torch.zeros((1, 40, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(lca.LcaError) as e:
        lca.compress_append(lay, kv, g, ik, ik)          # ring 32 < 40 + 16 - 1
    assert e.value.code == -3
    assert int(lay.seq_len[0]) == 0 and lay.len_max == 0
    with pytest.raises(lca.LcaError) as e:
        lca.indexer_topk(lay, torch.zeros((1, 1, 4, 64), device="cuda"),
                         torch.zeros((1, 1, 4), device="cuda"), 8)   # n_q > shortest row
    assert e.value.code == -1


@pytest.mark.parametrize("kind,n_q", [("csa", 1), ("csa", 64), ("hca", 1)], ids=["csa_decode", "csa_chunk", "hca"])
def test_graph_replay_matches_eager(kind, n_q):
    """The selection and attention calls captured in a HIP graph and replayed
    three times, with eager launches of the same calls between the replays:
    every replay gives the eager results bit for bit (no memset nodes in the
    graph; every call leaves its workspace ready for the next)."""
    lca = _lca()
    say("graph replay", kind, n_q)
    csa = kind == "csa"
    B, m, L, H, HI, k = 2, (4 if csa else 128), 20000, 64, 16, 256
    ref = SL.make_layer(91, "graph" + kind, B, m, 128, 256, int(csa), L // m + 8, [L, L - 5])
    Q = SL.queries(91, "graph" + kind, B, n_q, H, HI if csa else 0)
    lay = lca.Layer.from_host(ref)
    q = _dev(Q["q"])
    topk = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, n_q, H, 512), dtype=torch.float32, device="cuda")

    def step():
        if csa:
            lca.indexer_topk(lay, iq, iw, k, out=topk)
            lca.csa_attend(lay, q, topk, float(SCALE), out=out)
        else:
            lca.hca_attend(lay, q, float(SCALE), out=out)

    iq, iw = (_dev(Q["iq"]), _dev(Q["iw"])) if csa else (None, None)
    step()                                  # eager: allocates the workspaces
    torch.cuda.synchronize()
    t_ref, o_ref = topk.clone(), out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        topk.zero_()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert (not csa or torch.equal(topk, t_ref)) and torch.equal(out, o_ref), ("replay", rep)
        step()
        torch.cuda.synchronize()
        assert (not csa or torch.equal(topk, t_ref)) and torch.equal(out, o_ref), ("eager", rep)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_graph_replay_with_append(kind):
    """A whole decode step (append, then selection and attention for CSA, or
    attention over every entry for HCA) captured once with plans for the
    longest length it will reach, replayed six times; an eager twin of the
    layer takes the same six steps.  After every step the top-k lists, the
    outputs and the row lengths agree bit for bit, and so do the cache planes
    at the end.  The HCA rows cross a 128-token block boundary on the way."""
    lca = _lca()
    csa = kind == "csa"
    B, H, HI, k, steps = 2, 64, 16, 256, 6
    m, L = (4, 20001) if csa else (128, 128 * 40 - 3)
    say("graph replay with append", kind, B, L, steps)
    ref = SL.make_layer(92, "gapp" + kind, B, m, 128, 256, int(csa), (L + 64) // m + 8, [L, L - 6])
    tok = SL.tokens(92, "gapp" + kind, B, 1, 1)
    Q = SL.queries(92, "gapp" + kind, B, 1, H, HI)
    lg, le = lca.Layer.from_host(ref), lca.Layer.from_host(ref)
    d = {kk: _dev(v) for kk, v in tok.items()}
    iq, iw, q = _dev(Q["iq"]), _dev(Q["iw"]), _dev(Q["q"])
    bufs = {id(lay): (torch.empty((B, 1, k), dtype=torch.int32, device="cuda"),
                      torch.empty((B, 1, H, 512), dtype=torch.float32, device="cuda")) for lay in (lg, le)}

    def step(lay, plan_len=None):
        lca.compress_append(lay, d["kv"], d["gate"], d["ikey"], d["igate"])
        if plan_len is not None:
            lay.len_max = plan_len
        t, o = bufs[id(lay)]
        if csa:
            lca.indexer_topk(lay, iq, iw, k, out=t)
            lca.csa_attend(lay, q, t, float(SCALE), out=o)
        else:
            lca.hca_attend(lay, q, float(SCALE), out=o)

    final = L + steps + 2
    before = (lg.len_min, lg.len_max)
    lg.len_max = final                     # workspaces sized for the longest length
    if csa:
        lg.indexer_workspace(1, lca.indexer_workspace_bytes(lg, 1, HI, k))
    lg.workspace(lca.attend_workspace_bytes(lg, 1, H, k if csa else 0), "attend")
    lg.len_min, lg.len_max = before
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(lg, plan_len=final)
    torch.cuda.synchronize()
    lg.len_min, lg.len_max = before        # capture executes nothing
    for r in range(steps):
        g.replay()
        step(le)
        torch.cuda.synchronize()
        (tg, og), (te, oe) = bufs[id(lg)], bufs[id(le)]
        assert torch.equal(lg.seq_len, le.seq_len), r
        assert not csa or torch.equal(tg, te), r
        assert torch.equal(og, oe), r
    a, b = lg.download(), le.download()
    planes = ("nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv")
    for f in planes:
        if f in a:
            assert np.array_equal(a[f], b[f]), f
    assert int(b["seq_len"][0]) // m > L // m     # a block was finalised on the way


@pytest.mark.parametrize("n_q", [1, 20], ids=["decode", "chunk"])
def test_ratio1_csa_and_window_only(n_q):
    """Two layer variants on the same kernels: CSA at ratio 1 (the selection
    runs over the raw tokens, one block per token) through the indexer and
    the attention, and attention over the window alone (every list entry -1,
    as in a plain sliding-window layer)."""
    lca = _lca()
    B, lens, H, H_I, k, W = 2, [3000, 2411], 64, 16, 256, 128
    say("ratio-1 CSA and window-only", "n_q", n_q, "lens", lens)
    ref = SL.make_layer(6100 + n_q, "r1", B, 1, W, 256, 1, max(lens) + 8, lens)
    Q = SL.queries(6100 + n_q, "r1", B, n_q, H, H_I)
    lay = lca.Layer.from_host(ref)
    topk = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
    torch.cuda.synchronize()
    want_idx = oracle.indexer_topk(ref, Q["iq"], Q["iw"], k)
    assert np.array_equal(topk.cpu().numpy(), want_idx)
    got = lca.csa_attend(lay, _dev(Q["q"]), topk, float(SCALE))
    torch.cuda.synchronize()
    assert attn_rel_err(got.cpu().numpy(), oracle.csa_attend(ref, Q["q"], want_idx, SCALE)) <= ATTN_TOL
    none = np.full((B, n_q, 64), -1, np.int32)
    got = lca.csa_attend(lay, _dev(Q["q"]), _dev(none), float(SCALE))
    torch.cuda.synchronize()
    assert attn_rel_err(got.cpu().numpy(), oracle.csa_attend(ref, Q["q"], none, SCALE)) <= ATTN_TOL


# ------------------------------------------------------------------ status word

def _range_layer(lca, csa, seed):
    B, L, W = 2, 3000, 128
    m = 4 if csa else 128
    ref = SL.make_layer(seed, "rng", B, m, W, 256, int(csa), L // m + 8, [L, L - 5])
    return ref


FP16_RANGE_CASES = {   # case -> whether it sets LCA_STATUS_FP16_RANGE
    "none": False, "edges": False, "q_subnormal": False, "window_subnormal": False, "q_zero_head": False,
    "q_big": True, "q_tiny_head": True, "window_big": True, "window_tiny_group": True,
    "rope_big": True, "rope_tiny_group": True, "scale_big": True, "scale_small": True}


def _tiny_bits(seed, n):
    """bf16 bits of n values ~N(0,1) * 2^-20, all below 2^-14, some of which
    fp16 rounds (bits below its subnormal spacing 2^-24)."""
    v = synth.bf16_to_f32(synth.bf16_normal(seed, "tiny", (n,), "rng")) * np.float32(2.0 ** -20)
    bits = synth.bf16_bits(v)
    f = synth.bf16_to_f32(bits)
    assert np.abs(f).max() < 2.0 ** -14
    assert (f.astype(np.float16).astype(np.float32) != f).any()
    return bits


@pytest.mark.parametrize("what", list(FP16_RANGE_CASES))
@pytest.mark.parametrize("csa", [0, 1], ids=["hca", "csa"])
def test_attend_fp16_range_reported(what, csa):
    """Inputs the fp16 images may not hold to 2^-11 of their vector's largest
    magnitude set LCA_STATUS_FP16_RANGE: a query head or a 64-channel key
    group whose largest magnitude is above 65504 or nonzero and below 2^-14,
    FP8 scales outside [2^-14, 2^8).  In-range inputs leave the word clear:
    fp16's exact edges (65280, 2^-24, scales 2^-14 and just below 2^8), a
    value below fp16's subnormal spacing inside a vector of ordinary
    magnitude, an all-zero query head."""
    lca = _lca()
    say("attend fp16 range", what, "csa", csa)
    ref = _range_layer(lca, csa, 6200 + csa)
    Q = SL.queries(6200, "rng", 2, 1, 16)
    q = Q["q"].copy()
    m = ref["ratio"]
    p = int(ref["seq_len"][0]) - 1
    slot = p % ref["ring"]
    slot1 = (int(ref["seq_len"][1]) - 4) % ref["ring"]     # inside row 1's window
    b_last = (p + 1) // m - 1
    f32 = lambda v: synth.bf16_bits(np.array([v], np.float32))[0]
    if what == "q_big":
        q[0, 0, 3, 17] = f32(70144.0)
    elif what == "q_subnormal":
        q[1, 0, 0, 5] = f32(3e-8)              # below fp16's smallest subnormal 2^-24
    elif what == "q_zero_head":
        q[0, 0, 5, :] = 0
    elif what == "q_tiny_head":
        q[1, 0, 2, :] = _tiny_bits(1, 512)
    elif what == "window_big":
        ref["ring_kv"][0, slot, 100] = f32(-1.0e5)
    elif what == "window_subnormal":
        ref["ring_kv"][1, slot1, 480] = f32(1.5 * 2.0 ** -25)
    elif what == "window_tiny_group":
        ref["ring_kv"][1, slot1, 128:192] = _tiny_bits(2, 64)
    elif what == "rope_big":
        ref["rope"][0, b_last, 7] = f32(2.0 ** 17)
    elif what == "rope_tiny_group":
        ref["rope"][0, b_last, :] = _tiny_bits(3, 64)
    elif what == "scale_big":
        ref["kv_scale"][0, b_last, 2] = np.float32(300.0)
    elif what == "scale_small":
        ref["kv_scale"][1, 3, 0] = np.float32(1e-5)
    elif what == "edges":
        q[0, 0, 1, 2] = f32(65280.0)
        q[0, 0, 1, 3] = f32(2.0 ** -24)
        ref["ring_kv"][0, slot, 9] = f32(-65280.0)
        ref["kv_scale"][0, b_last, 1] = np.float32(2.0 ** -14)
        ref["kv_scale"][0, b_last, 3] = np.float32(255.0)
    lay = lca.Layer.from_host(ref)
    if csa:
        # blocks 0..62 and row 0's last block (not yet visible to row 1)
        sel = np.append(np.arange(63, dtype=np.int32), np.int32(b_last))
        topk = np.ascontiguousarray(np.broadcast_to(sel, (2, 1, 64)))
        lca.csa_attend(lay, _dev(q), _dev(topk), float(SCALE))
    else:
        lca.hca_attend(lay, _dev(q), float(SCALE))
    torch.cuda.synchronize()
    expect = FP16_RANGE_CASES[what]
    assert lay.status() == (lca.STATUS_FP16_RANGE if expect else 0), (what, lay.status())


def test_capacity_beyond_the_plan_is_reported():
    """Host mirrors below the device lengths stand for a graph replayed past
    its plan: each kernel keeps to its plan and sets its status bit; the
    compressor skips a block past max_blocks."""
    lca = _lca()
    say("capacity status")
    B, L, H, H_I, k = 2, 20000, 16, 4, 64
    ref = SL.make_layer(6300, "cap", B, 4, 128, 256, 1, L // 4 + 8, [L, L - 3])
    Q = SL.queries(6300, "cap", B, 1, H, H_I)
    for fused in (1, 0):
        lay = lca.Layer.from_host(ref)
        lay.len_min, lay.len_max = 9000, 10000          # plans for 2500 blocks
        lca.set_tuning("LCA_TOPK_FUSED", fused)
        try:
            lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
        finally:
            lca.set_tuning("LCA_TOPK_FUSED", None)
        torch.cuda.synchronize()
        assert lay.status() == lca.STATUS_INDEXER_CAPACITY, (fused, lay.status())
    href = SL.make_layer(6301, "caph", B, 128, 128, 256, 0, L // 128 + 8, [L, L - 3])
    lay = lca.Layer.from_host(href)
    lay.len_min, lay.len_max = 9000, 10000
    lca.set_tuning("LCA_ATTEND_SPLITS", 4)
    try:
        lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
    finally:
        lca.set_tuning("LCA_ATTEND_SPLITS", None)
    torch.cuda.synchronize()
    assert lay.status() == lca.STATUS_ATTEND_CAPACITY, lay.status()
    # compressor: 10 blocks fit, the device rows already hold 40 tokens
    cref = SL.make_layer(6302, "capc", 1, 4, 8, 32, 0, 10, [40])
    lay = lca.Layer.from_host(cref)
    before = lay.download()
    lay.len_min = lay.len_max = 0
    tok = SL.tokens(6302, "capc", 1, 4, 0)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]))
    torch.cuda.synchronize()
    after = lay.download()
    assert lay.status() == lca.STATUS_COMPRESS_CAPACITY, lay.status()
    assert int(after["seq_len"][0]) == 44
    for f in ("nope", "rope", "kv_scale"):
        assert np.array_equal(after[f], before[f]), f
