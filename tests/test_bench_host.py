"""Host-side figures of bench.py: the per-step algorithmic bytes and flops
that the roofline fractions divide by, checked against sums worked out by
hand from the per-unit costs (a 604-byte entry, a 34-byte indexer key, a
1024-byte window token, q and out at 1024 and 2048 bytes per head, 260 bytes
of indexer query and weight per indexer head, two 4-byte index passes per
selected block)."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))

import bench  # noqa: E402


def test_csa_decode_128k_bytes():
    wl = bench.WORKLOADS["csa_decode_128k"]
    per_row = (128 * 1024 + 64 * 1024 + 64 * 2048       # window, q, out
               + 32768 * 34 + 16 * 260                   # every indexer key, iq + iw
               + 2 * 512 * 4 + 512 * 604)                # top-k indices, selected entries
    assert per_row == 1_759_296
    assert bench.algorithmic_bytes(wl) == 32 * per_row == 56_297_472
    assert bench.dominant_bytes(wl) == 32 * (32768 * 34 + 16 * 260) == 35_784_704


def test_hca_decode_1m_bytes():
    wl = bench.WORKLOADS["hca_decode_1m"]
    per_row = 8192 * 604 + 128 * 1024 + 64 * 1024 + 64 * 2048
    assert bench.algorithmic_bytes(wl) == 16 * per_row == 84_410_368
    assert bench.dominant_bytes(wl) == bench.algorithmic_bytes(wl)


def test_prefill_chunk_counts():
    # 4096 queries at positions 262144 .. 266239 see 65536 + floor(j / 4)
    # blocks (j = 1 .. 4096): 3 zeros, four of each t = 1 .. 1023, then 1024
    extra = 4 * (1023 * 1024 // 2) + 1024
    flops, pairs = bench.prefill_score_flops(262144, 4096, 4, 16)
    assert pairs == 4096 * 65536 + extra == 270_531_584
    assert flops == pairs * 16 * 64 * 2
    # every query attends 512 listed blocks (all visible) and 128 window tokens
    assert bench.prefill_attend_flops(262144, 4096, 4, 64, 512, 128) == 4096 * 640 * 64 * 2 * 512 * 2
    # HCA: query i sees 2048 + floor((i + 1) / 128) blocks and 128 window
    # tokens; floor(j / 128) over j = 1 .. 4096 is 127 zeros, 128 of each
    # t = 1 .. 31, then 32
    hca_keys = 4096 * (2048 + 128) + 128 * (31 * 32 // 2) + 32
    assert bench.prefill_attend_flops(262144, 4096, 128, 64, 262144 // 128 + 4096, 128) == hca_keys * 64 * 2 * 512 * 2
