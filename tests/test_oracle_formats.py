"""Pins of the oracle's number formats (CPU only).

They tie the oracle's codecs to the public format tables (golden/formats.json),
to exhaustive round trips, to every rounding midpoint, and to PyTorch's own
bf16 and float8_e4m3fn conversions (library routines) on random inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))


def _val(v):
    return float("nan") if v == "nan" else float(v)


def test_e4m3_table_points():
    for row in GOLD["e4m3"]:
        got = oracle.e4m3_value(row["code"])
        want = _val(row["value"])
        if math.isnan(want):
            assert math.isnan(got), row
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), row


def test_e4m3_monotone_and_count():
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert len(set(vals)) == 127 and max(vals) == 448.0


def test_e4m3_roundtrip_every_code():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)


def test_e4m3_midpoints_round_to_even_and_saturate():
    for c in range(0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        assert np.float32(mid) == mid
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == want, hex(c)
        assert oracle.e4m3_encode(-mid) == 0x80 | want
        # just off the midpoint
        assert oracle.e4m3_encode(float(np.nextafter(np.float32(mid), np.float32(0)))) == c
        assert oracle.e4m3_encode(float(np.nextafter(np.float32(mid), np.float32(1e9)))) == c + 1
    for x in (448.0, 449.0, 463.9, 464.0, 500.0, 1e30, float("inf")):
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], np.uint8)
    # compare decoded values (+0 and -0 are equal)
    gv = np.array([oracle.e4m3_value(c) for c in got])
    rv = np.array([oracle.e4m3_value(c) for c in ref])
    assert np.array_equal(gv, rv)


def test_e2m1_table_and_rounding():
    for row in GOLD["e2m1"]:
        assert oracle.e2m1_value(row["code"]) == row["value"]
    for row in GOLD["e2m1_rounding"]:
        assert oracle.e2m1_encode(row["x"]) == row["code"], row
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert oracle.e2m1_value(oracle.e2m1_encode(v)) == v


def test_e8m0_and_bf16_points():
    for row in GOLD["e8m0"]:
        got, want = oracle.e8m0_value(row["byte"]), _val(row["value"])
        assert (math.isnan(got) and math.isnan(want)) or got == want
    for row in GOLD["bf16"]:
        assert oracle.bf16_encode(row["x"]) == row["bits"], row


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-20, 20, 50000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_fp8_group_scale_and_extremes():
    rng = np.random.default_rng(11)
    for trial in range(50):
        y = (rng.standard_normal(64) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        codes, s = oracle.fp8_group_quant(y)
        amax = np.abs(y).max()
        assert s == np.float32(amax) / np.float32(448.0)
        i = int(np.abs(y).argmax())
        assert codes[i] & 0x7F == 0x7E            # the amax element hits +-448
        deq = np.array([oracle.e4m3_value(c) for c in codes]) * s
        # 3 mantissa bits: relative error <= 2^-4 for normal codes (plus the
        # subnormal step 2^-9 * s in absolute terms)
        assert np.all(np.abs(deq - y) <= 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * s + 1e-30)
    codes, s = oracle.fp8_group_quant(np.zeros(64, np.float32))
    assert s == 0.0 and not codes.any()


def test_mxfp4_block_rules():
    # amax 1.0 -> shared exponent floor(log2 1) - 2 = -2 (byte 125); 1.0 -> 4 -> code 6
    y = np.zeros(32, np.float32)
    y[0] = 1.0
    y[3] = -0.25
    packed, e = oracle.mxfp4_quant(y)
    assert e == 125
    assert packed[0] & 0xF == 6               # element 0 in the low nibble of byte 0
    assert packed[1] >> 4 == 0x8 | 2          # element 3: -0.25 * 4 = -1.0 -> code 0b1010
    # amax 7 -> exponent 0 (byte 127), 7 saturates to 6
    y = np.zeros(32, np.float32)
    y[31] = 7.0
    packed, e = oracle.mxfp4_quant(y)
    assert e == 127 and packed[15] >> 4 == 7
    packed, e = oracle.mxfp4_quant(np.zeros(32, np.float32))
    assert e == 0 and not packed.any()
    # dequantized block is within half a step of the input, elementwise
    rng = np.random.default_rng(5)
    for _ in range(50):
        y = rng.standard_normal(32).astype(np.float32) * 3
        packed, e = oracle.mxfp4_quant(y)
        sc = oracle.e8m0_value(e)
        nib = np.stack([packed & 0xF, packed >> 4], 1).reshape(-1)
        deq = np.array([oracle.e2m1_value(c) for c in nib]) * sc
        step = np.where(np.abs(y) / sc < 2, 0.5, np.where(np.abs(y) / sc < 4, 1.0, 2.0)) * sc
        sat = np.maximum(0.0, np.abs(y) - 6 * sc)   # beyond 6 * scale it saturates
        assert np.all(np.abs(deq - y) <= step / 2 + sat + 1e-7)
