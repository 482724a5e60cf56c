"""Pins of the oracle's compressor, indexer, top-k and attention (CPU only).

Each check ties the oracle to something other than itself: a hand-derived
closed form (golden/closed_forms.json), an invariant of softmax pooling or
softmax attention, an exact-rational brute force, or a brute-force sort.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import layers as SL
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
FMT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))
E2M1 = {r["code"]: Fraction(r["value"]).limit_denominator(4) for r in FMT["e2m1"]}
for c in range(8):
    E2M1.setdefault(c, Fraction([0, 1, 2, 3, 4, 6, 8, 12][c], 2))
    E2M1.setdefault(c | 8, -E2M1[c])
SCALE = np.float32(1.0 / math.sqrt(512.0))


def ulp32(x):
    x = np.float32(abs(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x)


def round_f32(fr: Fraction) -> float:
    """Correctly rounded (RNE) conversion of an exact rational to binary32."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** max(e - 23, -149)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


# ------------------------------------------------------------------ compressor

def test_pool_closed_form_m2():
    g = GOLD["pool_m2"]
    y = oracle.pool(np.array(g["x"]), np.array(g["gate"]), np.array(g["bias"]))
    for got, want in zip(y, g["y"]):
        assert abs(got - want) <= 4 * ulp32(want)


def test_pool_ratio_one_is_identity_bitwise():
    rng = np.random.default_rng(1)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((1, 512))))
    z = rng.standard_normal((1, 512)).astype(np.float32) * 5
    b = rng.standard_normal((1, 512)).astype(np.float32)
    y = oracle.pool(x, z, b)
    assert np.array_equal(y.view(np.uint32), x[0].view(np.uint32))


@pytest.mark.parametrize("m", [2, 4, 128])
def test_pool_identical_tokens_and_convexity_and_shift(m):
    rng = np.random.default_rng(m)
    tok = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal(512)))
    x = np.tile(tok, (m, 1))
    z = rng.standard_normal((m, 512)).astype(np.float32)
    b = rng.standard_normal((m, 512)).astype(np.float32)
    y = oracle.pool(x, z, b)
    # the weights sum to 1 up to rounding: |y - x| <= 2 m u |x| (u = 2^-24)
    assert np.all(np.abs(y - tok) <= 2 * m * 2.0 ** -24 * np.abs(tok))
    # the double-precision pool gives it back to within its own rounding bound
    y64 = oracle.pool(x, z, b, double=True)
    assert np.all(np.abs(y64 - tok) <= 4 * m * 2.0 ** -53 * np.abs(tok))
    # convex combination of distinct tokens
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((m, 512))))
    y = oracle.pool(x, z, b)
    lo, hi = x.min(0), x.max(0)
    tol = 2 * m * 2.0 ** -24 * np.maximum(np.abs(lo), np.abs(hi))
    assert np.all(y >= lo - tol) and np.all(y <= hi + tol)
    # shifting all logits of a channel leaves the pooled value unchanged
    y2 = oracle.pool(x, z + np.float32(3.0), b)
    assert np.allclose(y2, y, rtol=1e-5, atol=1e-6)


def test_pool_f32_close_to_f64():
    rng = np.random.default_rng(2)
    for m in (4, 128):
        x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((m, 512))))
        z = rng.standard_normal((m, 512)).astype(np.float32)
        b = rng.standard_normal((m, 512)).astype(np.float32)
        y32 = oracle.pool(x, z, b).astype(np.float64)
        y64 = oracle.pool(x, z, b, double=True)
        assert np.linalg.norm(y32 - y64) <= 1e-5 * np.linalg.norm(y64)


def _compress_layer(m, has_idx, R=64, W=16, MB=64, B=2):
    L = SL.empty_layer(B, m, W, R, has_idx, MB)
    L["pos_bias"], L["ipos_bias"] = SL.pos_bias(5, "t", m, has_idx)
    return L


@pytest.mark.parametrize("m,has_idx", [(4, 1), (8, 0), (1, 1)])
def test_chunked_equals_token_by_token(m, has_idx):
    T = 37
    toks = SL.tokens(9, "c", 2, T, has_idx)
    A = _compress_layer(m, has_idx)
    Bc = _compress_layer(m, has_idx)
    oracle.compress_append(A, toks["kv"], toks["gate"], toks.get("ikey"), toks.get("igate"))
    for t in range(T):
        sl = slice(t, t + 1)
        oracle.compress_append(Bc, toks["kv"][:, sl].copy(), toks["gate"][:, sl].copy(),
                               toks["ikey"][:, sl].copy() if has_idx else None,
                               toks["igate"][:, sl].copy() if has_idx else None)
    for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv", "ring_gate",
              "ring_ikey", "ring_igate"):
        assert np.array_equal(A[f], Bc[f]), f
    nb = T // m
    assert np.all(A["seq_len"] == T)
    # blocks are aligned at position 0: exactly floor(T/m) entries written, and
    # entry b is the quantized pool of tokens bm .. bm+m-1
    for row in range(2):
        for b in range(nb):
            x = synth.bf16_to_f32(toks["kv"][row, b * m:(b + 1) * m])
            y = oracle.pool(x, toks["gate"][row, b * m:(b + 1) * m], A["pos_bias"])
            nope, rope, sc = oracle.make_entry(y)
            assert np.array_equal(A["nope"][row, b], nope)
            assert np.array_equal(A["rope"][row, b], rope)
            assert np.array_equal(A["kv_scale"][row, b], sc)
        assert not A["nope"][row, nb:].any()


# ------------------------------------------------------------------ indexer

def _exact_dot(qcode, qe, kcode, ke, h):
    """The exact rational dot product of head h's dequantized MXFP4 query with
    the dequantized MXFP4 key (e2m1 values from the format table times the
    E8M0 powers of two)."""
    dot = Fraction(0)
    for el in range(64):
        j = el // 32
        qb, kb = int(qcode[h, el // 2]), int(kcode[el // 2])
        qn = (qb >> 4) if el & 1 else (qb & 15)
        kn = (kb >> 4) if el & 1 else (kb & 15)
        sc = Fraction(2) ** (int(qe[h, j]) - 127 + int(ke[j]) - 127)
        dot += E2M1[qn] * E2M1[kn] * sc
    return dot


def _brute_score(qcode, qe, w, kcode, ke):
    """Exact-rational brute force of the defined evaluation order: per head
    the exact dot rounded once to binary32, ReLU, then one chain of fused
    multiply-adds (each rounded once) over the heads in ascending order from
    +0."""
    score = 0.0
    for h in range(len(w)):
        d = round_f32(_exact_dot(qcode, qe, kcode, ke, h))
        r = d if d > 0 else 0.0
        score = round_f32(Fraction(float(np.float32(w[h]))) * Fraction(r) + Fraction(score))
    return score + 0.0


def test_index_score_closed_form():
    qf = np.zeros((2, 64), np.float32)
    qf[0, 0] = 1.0
    qf[1, 33] = -2.0
    qcode = np.zeros((2, 32), np.uint8)
    qe = np.zeros((2, 2), np.uint8)
    for h in range(2):
        qcode[h], qe[h] = oracle.make_idx(qf[h])
    kcode = np.zeros(32, np.uint8)
    kcode[0] = 0x07                     # element 0 = 6 (low nibble)
    kcode[16] = 0x50                    # element 33 = 3 (high nibble of byte 16)
    ke = np.array([127, 128], np.uint8)
    s, inexact = oracle.index_score(qcode, qe, np.array([0.5, 2.0], np.float32), kcode, ke)
    assert not inexact and s == GOLD["index_score"]["score"]


def _random_query_key(rng, H):
    qf = rng.standard_normal((H, 64)).astype(np.float32) * 10.0 ** rng.uniform(-2, 2)
    qcode = np.zeros((H, 32), np.uint8)
    qe = np.zeros((H, 2), np.uint8)
    for h in range(H):
        qcode[h], qe[h] = oracle.make_idx(qf[h])
    kcode = rng.integers(0, 256, 32).astype(np.uint8)
    ke = (127 + rng.integers(-6, 6, 2)).astype(np.uint8)
    return qcode, qe, kcode, ke


def test_index_score_matches_exact_rational_brute_force():
    rng = np.random.default_rng(17)
    for trial in range(48):
        H = int(rng.integers(1, 6)) if trial < 16 else int(rng.integers(7, 33))
        qcode, qe, kcode, ke = _random_query_key(rng, H)
        w = rng.standard_normal(H).astype(np.float32)      # any sign
        s, inexact = oracle.index_score(qcode, qe, w, kcode, ke)
        assert not inexact
        want = _brute_score(qcode, qe, w, kcode, ke)
        assert np.float32(s).view(np.uint32) == np.float32(want).view(np.uint32), (trial, s, want)


def test_index_score_close_to_exact_weighted_sum():
    """Order-free pin: the score is the exact sum over heads of
    w_h * ReLU(dot_h) (dot_h the exactly rounded dot) up to the rounding of
    H fused multiply-adds, |err| <= H u / (1 - H u) * sum_h |w_h r_h|, u = 2^-24.
    A dropped head, a wrong weight index or a sign error breaks it."""
    rng = np.random.default_rng(18)
    u = 2.0 ** -24
    for trial in range(60):
        H = int(rng.integers(1, 33))
        qcode, qe, kcode, ke = _random_query_key(rng, H)
        w = rng.standard_normal(H).astype(np.float32)
        if trial % 3 == 0:
            w = np.abs(w)
        elif trial % 3 == 1:
            w = -np.abs(w)
        s, _ = oracle.index_score(qcode, qe, w, kcode, ke)
        terms = []
        for h in range(H):
            d = Fraction(round_f32(_exact_dot(qcode, qe, kcode, ke, h)))
            terms.append(Fraction(float(w[h])) * max(d, Fraction(0)))
        exact = sum(terms, Fraction(0))
        bound = Fraction(H) * Fraction(u) / (1 - H * Fraction(u)) * sum(abs(t) for t in terms)
        assert abs(Fraction(float(s)) - exact) <= bound, (trial, s, float(exact))
        if all(t >= 0 for t in terms) or all(t <= 0 for t in terms):
            # one-signed terms: the relative error is at most the same factor
            assert abs(Fraction(float(s)) - exact) <= bound


def test_index_score_negative_weights_and_zero():
    """All-negative weights give negative (or +0) scores; a score that is
    zero is +0 whatever the weights' signs."""
    rng = np.random.default_rng(19)
    for trial in range(20):
        H = int(rng.integers(1, 17))
        qcode, qe, kcode, ke = _random_query_key(rng, H)
        w = -np.abs(rng.standard_normal(H).astype(np.float32))
        s, _ = oracle.index_score(qcode, qe, w, kcode, ke)
        assert s <= 0.0
        if s == 0.0:
            assert np.float32(s).view(np.uint32) == 0
    # every dot negative -> every ReLU +0 -> score +0 even with w < 0
    qcode = np.zeros((2, 32), np.uint8)
    qe = np.full((2, 2), 127, np.uint8)
    qcode[:, 0] = 0x02                       # element 0 = +1.0
    kcode = np.zeros(32, np.uint8)
    kcode[0] = 0x0A                          # element 0 = -1.0
    s, _ = oracle.index_score(qcode, qe, np.array([-1.0, -2.0], np.float32), kcode,
                              np.array([127, 127], np.uint8))
    assert np.float32(s).view(np.uint32) == 0


def test_topk_brute_force_ties_and_padding():
    rng = np.random.default_rng(4)
    for n, k in [(100, 10), (50, 50), (30, 64), (0, 4), (257, 31)]:
        s = rng.standard_normal(n).astype(np.float32)
        s[rng.integers(0, max(n, 1), n // 3)] = 0.5          # ties
        s[: n // 5] = np.abs(s[: n // 5])
        got = oracle.topk_select(s, k)
        order = sorted(range(n), key=lambda b: (-float(s[b]), b))[: min(k, n)]
        want = sorted(order) + [-1] * (k - min(k, n))
        assert list(got) == want
    # equal scores go to the lowest indices
    got = oracle.topk_select(np.ones(20, np.float32), 5)
    assert list(got) == [0, 1, 2, 3, 4]
    # negative scores are ordered correctly
    got = oracle.topk_select(np.array([-3, -1, -2, -5], np.float32), 2)
    assert list(got) == [1, 2]


def test_needles_are_selected_with_margin():
    seed, m, W, H_I, k = 1001, 4, 128, 4, 64
    L = SL.make_layer(seed, "csa", 1, m, W, 256, 1, 1024, [4096])
    Q = SL.queries(seed, "csa", 1, 1, 16, H_I)
    needles = SL.plant_needles(L, seed, "csa", 0, 4, Q["iq"][0, 0], Q["iw"][0, 0], Q["q"][0, 0])
    top = oracle.indexer_topk(L, Q["iq"], Q["iw"], k)[0, 0]
    assert set(needles) <= set(top.tolist())
    sc = oracle.indexer_scores(L, 0, 0, 1, Q["iq"], Q["iw"])
    others = np.sort(np.delete(sc, needles))[::-1]
    kth = others[k - len(needles) - 1]
    assert sc[needles].min() >= 1.01 * kth


def test_indexer_visibility_rule():
    # a query at position p sees blocks b < floor((p+1)/m) only
    m = 4
    L = SL.make_layer(3, "v", 1, m, 8, 64, 1, 64, [30])   # 30 tokens -> 7 blocks
    Q = SL.queries(3, "v", 1, 3, 4, 4)
    for qi, p in enumerate((27, 28, 29)):
        sc = oracle.indexer_scores(L, 0, qi, 3, Q["iq"], Q["iw"])
        assert len(sc) == (p + 1) // m


# ------------------------------------------------------------------ attention

def test_attend_two_keys_closed_form():
    keys = np.zeros((2, 512))
    keys[0, 0] = 1.0
    keys[1, 1] = 1.0
    q = np.zeros((1, 512), np.uint16)
    q[0, 1] = oracle.bf16_encode(2.0)
    scale = math.log(3.0) / 2.0
    out = oracle.attend_keys(q, keys, scale)
    want = GOLD["attend_two_keys"]["out"]
    assert abs(out[0, 0] - want[0]) < 1e-6 and abs(out[0, 1] - want[1]) < 1e-6
    assert not out[0, 2:].any()


def test_attend_single_key_zero_query_identical_keys():
    rng = np.random.default_rng(8)
    key = rng.standard_normal(512)
    q = synth.bf16_bits(rng.standard_normal((3, 512)))
    out = oracle.attend_keys(q, key[None, :], SCALE)
    assert np.allclose(out, np.float32(key)[None, :], rtol=0, atol=1e-6 * np.abs(key).max())
    keys = rng.standard_normal((7, 512))
    out = oracle.attend_keys(np.zeros((1, 512), np.uint16), keys, SCALE)
    assert np.allclose(out[0], keys.mean(0), atol=1e-6)
    out = oracle.attend_keys(q, np.tile(key, (9, 1)), SCALE)
    assert np.allclose(out, np.float32(key)[None, :], atol=1e-6 * np.abs(key).max())


def _marker_channel(b):
    return (b * 67) % 448


def _marker_layer(m, W, R, MB, length):
    """Entries and window tokens that are one-hot markers, so that with q = 0
    the output is the uniform mean over exactly the key set."""
    L = SL.empty_layer(1, m, W, R, 1, MB)
    L["pos_bias"], L["ipos_bias"] = SL.pos_bias(1, "mk", m, 1)
    L["seq_len"][0] = length
    one = 0x38                                          # e4m3 1.0
    for b in range(length // m):
        L["nope"][0, b, _marker_channel(b)] = one
        L["kv_scale"][0, b, :7] = 0.25 * np.arange(1, 8)  # group g scales by (g+1)/4
    for t in range(max(0, length - R), length):
        L["ring_kv"][0, t % R, 448 + (t % 64)] = oracle.bf16_encode(1.0)
    return L


def test_hca_key_set_visibility_and_window():
    m, W, R = 4, 3, 16
    L = _marker_layer(m, W, R, 32, 22)                  # positions 0..21
    q = np.zeros((1, 3, 2, 512), np.uint16)             # queries at p = 19, 20, 21
    out = oracle.hca_attend(L, q, SCALE)
    for qi, p in enumerate((19, 20, 21)):
        nv = (p + 1) // m
        nk = nv + W
        o = out[0, qi, 0]
        chans = [_marker_channel(b) for b in range(nv)]
        for c in chans:                                 # entry value 1.0 * scale of its 64-group
            assert abs(o[c] - 0.25 * (c // 64 + 1) / nk) < 1e-7
        assert np.count_nonzero(o[:448]) == nv
        for t in range(p - W + 1, p + 1):
            assert abs(o[448 + t % 64] - 1.0 / nk) < 1e-7
        assert np.count_nonzero(o[448:]) == W
        assert np.array_equal(out[0, qi, 0], out[0, qi, 1])


def test_csa_with_all_blocks_equals_hca_bitwise():
    seed = 12
    L = SL.make_layer(seed, "eq", 2, 4, 16, 64, 1, 64, [150, 97])
    Q = SL.queries(seed, "eq", 2, 2, 4)
    k = 64
    topk = np.full((2, 2, k), -1, np.int32)
    for b in range(2):
        for qi in range(2):
            p = L["seq_len"][b] - 2 + qi
            nv = (p + 1) // 4
            topk[b, qi, :nv] = np.arange(nv)
    a = oracle.csa_attend(L, Q["q"], topk, SCALE)
    h = oracle.hca_attend(L, Q["q"], SCALE)
    assert np.array_equal(a.view(np.uint32), h.view(np.uint32))


def test_csa_ignores_padding_and_invisible_indices():
    seed = 13
    L = SL.make_layer(seed, "pad", 1, 4, 16, 64, 1, 64, [120])
    Q = SL.queries(seed, "pad", 1, 1, 4)
    base = np.array([[[3, 7, 11, -1, -1]]], np.int32)
    nv = (120 - 1 + 1) // 4                               # query at p = 119 sees 30 blocks
    junk = np.array([[[3, 7, 11, nv, 60]]], np.int32)     # block nv is not yet complete
    a = oracle.csa_attend(L, Q["q"], base, SCALE)
    b = oracle.csa_attend(L, Q["q"], junk, SCALE)
    assert np.array_equal(a, b)


def test_decode_equals_prefill_row():
    seed, m, W, R = 21, 4, 8, 64
    T = 40
    toks = SL.tokens(seed, "dp", 1, T, 1)
    Q = SL.queries(seed, "dp", 1, T, 4)
    full = _compress_layer(m, 1, R=R, W=W, MB=16, B=1)
    oracle.compress_append(full, toks["kv"], toks["gate"], toks["ikey"], toks["igate"])
    pre = oracle.hca_attend(full, Q["q"], SCALE)          # n_q = T: every position
    for p in (0, 3, 4, 17, 39):
        part = _compress_layer(m, 1, R=R, W=W, MB=16, B=1)
        oracle.compress_append(part, toks["kv"][:, : p + 1].copy(), toks["gate"][:, : p + 1].copy(),
                               toks["ikey"][:, : p + 1].copy(), toks["igate"][:, : p + 1].copy())
        dec = oracle.hca_attend(part, Q["q"][:, p:p + 1].copy(), SCALE)
        assert np.array_equal(dec[0, 0], pre[0, p])


def test_kv_bytes_per_token_ratio():
    g = GOLD["kv_bytes_per_token"]
    csa = (g["csa_entry_bytes"] + g["idx_key_bytes"]) / g["csa_ratio"]
    hca = g["csa_entry_bytes"] / g["hca_ratio"]
    ratio = (csa + hca) / 2 / g["gqa_bytes"]
    assert abs(ratio - g["expected_ratio"]) < 0.001
    # the entry layout the oracle writes: 448 codes + 64 bf16 + 7 fp32 scales
    assert 448 + 64 * 2 + 7 * 4 == g["csa_entry_bytes"]
    assert 32 + 2 == g["idx_key_bytes"]
