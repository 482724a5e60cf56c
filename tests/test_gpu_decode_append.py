"""The decode step's append and selection in one call
(lca_decode_append_topk) against the two calls it stands for
(lca_compress_append of one token per row, then lca_indexer_topk) on twin
layers built from one host image: after every step the top-k lists, the
row lengths and the status word agree bit for bit, and so does every cache
plane (ring, entries, indexer keys) after the steps.  The separate calls are
checked against the oracle in the compressor and indexer parity tests, so
this bit-for-bit equality carries that parity over.  Steps cross block
boundaries: a token that completes a block has that block's indexer key
scored in the same launch.
Shapes outside the one-launch plan (H_I > 16, the selection forced into a
launch of its own, blocks of more than 8 tokens) take the two launches and
must agree as well."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth import layers as SL

pytestmark = pytest.mark.gpu

PLANES = ("nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv", "ring_gate", "ring_ikey", "ring_igate",
          "seq_len")

# name, batch, lengths, ratio, H_I, k, steps, page blocks (0: contiguous), tuning
CASES = [
    ("ragged_h16_k512", 3, [9000, 4101, 6002], 4, 16, 512, 9, 0, {}),
    ("h4_k64", 2, [4093, 3000], 4, 4, 64, 9, 0, {}),
    ("ratio1_h8", 2, [3000, 2000], 1, 8, 100, 4, 0, {}),
    ("ratio8_h16", 1, [20001], 8, 16, 256, 17, 0, {}),
    ("k_ge_visible", 2, [203, 37], 4, 8, 64, 9, 0, {}),
    ("paged_pb256", 2, [30000, 12001], 4, 16, 512, 9, 256, {}),
    ("rows_128k", 4, [131071, 131072, 131069, 131070], 4, 16, 512, 5, 0, {}),
    ("two_launches_h32", 2, [5000, 3003], 4, 32, 128, 5, 0, {}),
    ("two_launches_forced", 2, [5000, 3003], 4, 16, 128, 5, 0, {"LCA_TOPK_FUSED": 0}),
    ("two_launches_ratio16", 1, [8000], 16, 16, 128, 17, 0, {}),
]


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


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_append_topk_matches_two_calls(case, tuning):
    lca = _lca()
    name, B, lens, m, HI, k, steps, PB, tune = case
    seed = 7100 + len(name)
    say("decode append", name, "B", B, "lens", lens, "ratio", m, "H_I", HI, "k", k, "steps", steps, "pb", PB,
        "seed", seed, "tuning", tune)
    for var, val in tune.items():
        tuning(var, val)
    MB = (max(lens) + steps) // m + 8
    if PB:
        MB = -(-MB // PB) * PB                 # whole pages
    ref = SL.make_layer(seed, name, B, m, 128, 256, 1, MB, lens)
    if PB:
        ref = SL.paginate(ref, seed, PB, reserve_blocks=steps // m + 2)
    one, two = lca.Layer.from_host(ref), lca.Layer.from_host(ref)
    finalised = 0
    for s in range(steps):
        tok = SL.tokens(seed, name, B, 1, 1, step=s)
        Q = SL.queries(seed, name, B, 1, 16, HI, step=s)
        d = {kk: _dev(v) for kk, v in tok.items()}
        iq, iw = _dev(Q["iq"]), _dev(Q["iw"])
        got = lca.decode_append_topk(one, d["kv"], d["gate"], d["ikey"], d["igate"], iq, iw, k)
        lca.compress_append(two, d["kv"], d["gate"], d["ikey"], d["igate"])
        want = lca.indexer_topk(two, iq, iw, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want), ("topk", s)
        assert torch.equal(one.seq_len, two.seq_len), ("seq_len", s)
        assert (one.len_min, one.len_max) == (two.len_min, two.len_max), ("mirrors", s)
        assert one.status() == two.status() == 0, ("status", s, one.status(), two.status())
        finalised += sum(int((L + s + 1) % m == 0) for L in lens)
    a, b = one.download(), two.download()
    for f in PLANES:
        if f in a:
            assert np.array_equal(a[f], b[f]), f
    assert finalised > 0                       # blocks completed on the way


def test_decode_append_rejects_hca_layer():
    lca = _lca()
    ref = SL.make_layer(7199, "hcarej", 1, 128, 128, 256, 0, 64, [4000])
    lay = lca.Layer.from_host(ref)
    tok = SL.tokens(7199, "hcarej", 1, 1, 1)
    Q = SL.queries(7199, "hcarej", 1, 1, 16, 4)
    d = {kk: _dev(v) for kk, v in tok.items()}
    with pytest.raises(lca.LcaError) as e:
        lca.decode_append_topk(lay, d["kv"], d["gate"], d["ikey"], d["igate"], _dev(Q["iq"]), _dev(Q["iw"]), 16)
    assert e.value.code == -1
    assert int(lay.seq_len[0]) == 4000 and lay.len_max == 4000
