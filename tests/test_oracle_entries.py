"""Pins of the oracle's entry packers (CPU only): orc_make_entry and
orc_make_idx against hand-worked entries (golden/entries.json), and the FP8
group rule code = e4m3(RN(x * RN(448 / amax))) against the alternative
e4m3(RN(x / scale)) on a case where the two differ.

The expected codes were derived by hand from the format definitions; the
test re-derives the rule-discriminating case with exact rationals (not with
the oracle) so that the stored derivation is itself checked.
"""
import json
import os
from fractions import Fraction

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "entries.json")))


def _f(hexbits):
    return np.array([int(hexbits, 16)], np.uint32).view(np.float32)[0]


def _vec(n, table):
    y = np.zeros(n, np.float32)
    for i, h in table.items():
        y[int(i)] = _f(h)
    return y


def test_make_entry_hand_worked():
    g = GOLD["kv_entry"]
    nope, rope, sc = oracle.make_entry(_vec(512, g["y"]))
    want = np.zeros(448, np.uint8)
    for i, h in g["codes"].items():
        want[int(i)] = int(h, 16)
    # compare decoded values (+0 and -0 are the same value); -0 is also
    # checked bit for bit where the hand-worked entry states it
    dv = lambda c: np.array([oracle.e4m3_value(int(x)) for x in c])
    assert np.array_equal(dv(nope), dv(want)), np.nonzero(dv(nope) != dv(want))
    assert nope[7] == 0x80
    assert np.array_equal(sc.view(np.uint32), np.array([int(h, 16) for h in g["scales"]], np.uint32))
    want_r = np.zeros(64, np.uint16)
    for i, h in g["rope_bits"].items():
        want_r[int(i) - 448] = int(h, 16)
    assert np.array_equal(rope, want_r)


def test_make_idx_hand_worked():
    for name in ("idx_key", "idx_key_clamped"):
        g = GOLD[name]
        code, e = oracle.make_idx(_vec(64, g["y"]))
        want = np.zeros(32, np.uint8)
        for i, h in g["code"].items():
            want[int(i)] = int(h, 16)
        assert np.array_equal(code, want), (name, code, want)
        assert [int(x) for x in e] == [int(h, 16) for h in g["e8m0"]], name


def _rn32(fr: Fraction) -> Fraction:
    """Exact rational rounded to the nearest binary32 (ties to even), normal range."""
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (e - 23)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (1 if fr > 0 else -1) * fl * q


def test_fp8_rule_multiplies_by_448_over_amax():
    """Group 3 of the hand-worked entry: x * (448/amax) lands just above an
    e4m3 midpoint while x / (amax/448) lands on it (a tie to the even code),
    so the rule is told apart from its plausible alternative."""
    amax = Fraction(float(_f("0x402fdc99")))
    x = Fraction(float(_f("0x3c558bdf")))
    inv = _rn32(448 / amax)
    s = _rn32(amax / 448)
    t_mul = _rn32(x * inv)
    t_div = _rn32(x / s)
    mid = Fraction(17, 8)                        # between e4m3 2.0 (0x40) and 2.25 (0x41)
    assert t_mul > mid and t_div == mid
    codes, scale = oracle.fp8_group_quant(_vec(64, {"0": "0x402fdc99", "1": "0x3c558bdf"}))
    assert codes[1] == 0x41                      # the x * (448/amax) rule; x / s would give 0x40
    assert Fraction(float(np.float32(scale))) == s
