"""GPU parity at the full workload sizes, checked on sampled rows / queries.

The GPU runs one step of each workload over every row with the same launches
as the benchmark (one append, the indexer, the attention); the oracle then
repeats the step for a few sampled rows (or, for the prefill chunk, a few
sampled queries) and every sampled output is held to the usual bar: entries
equal up to rounding-midpoint code flips, scores and top-k sets bit exact,
attention within 2e-3 (per-row max error over max magnitude).

Inputs come from synth (seeded); expected values come from the oracle only.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from synth import layers as SL

from gpu_helpers import (ATTN_TOL, attn_rel_err, check_indexer_keys, check_topk, compare_entries,
                         indexer_row_keys)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
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


def _ring_tokens(V, f, p0, n):
    """tokens p0 .. p0+n-1 of the one-row oracle view, from its ring: [1][n][C]"""
    slots = np.arange(p0, p0 + n) % V["ring"]
    return V[f][0][slots][None]


def _score_keys(lay, lca, n_q, H_I, k):
    """the indexer's workspace and its layout; the histograms must be zero"""
    ws = lay.indexer_workspace(n_q)
    layout = lca.indexer_layout(lay, n_q, H_I, k)
    assert not ws[:layout["zero"]].view(torch.int32).any().item()     # counters, histograms left zeroed
    return ws, layout


def _check_finalised(got, V, r, block, m, has_idx):
    flips = compare_entries(got, V, r, [block],
                            _ring_tokens(V, "ring_kv", block * m, m),
                            _ring_tokens(V, "ring_gate", block * m, m),
                            _ring_tokens(V, "ring_ikey", block * m, m) if has_idx else None,
                            _ring_tokens(V, "ring_igate", block * m, m) if has_idx else None,
                            V["pos_bias"], V.get("ipos_bias"), m)
    return flips


def test_csa_decode_128k_fullsize():
    """32 rows x 131072 tokens (32768 blocks), 64 heads, 16 indexer heads,
    k = 512, W = 128, 16 needles per row; the step finalises block 32767."""
    lca = _lca()
    B, ctx, m, H, HI, k, W, needles = 32, 131072, 4, 64, 16, 512, 128, 16
    seed, tag = 1001, "csa"
    say("csa_decode_128k fullsize B", B, "ctx", ctx, "seed", seed)
    ref = SL.make_layer(seed, tag, B, m, W, 256, 1, ctx // m + 64, [ctx - 1] * B)
    Q = SL.queries(seed, tag, B, 1, H, HI)
    planted = [SL.plant_needles(ref, seed, tag, b, needles, Q["iq"][b, 0], Q["iw"][b, 0], Q["q"][b, 0])
               for b in range(B)]
    tok = SL.tokens(seed, "fullsize_step", B, 1, 1)
    lay = lca.Layer.from_host(ref)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]), _dev(tok["ikey"]), _dev(tok["igate"]))
    topk = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
    out = lca.csa_attend(lay, _dev(Q["q"]), topk, float(SCALE))
    torch.cuda.synchronize()
    got_topk, got_out = topk.cpu().numpy(), out.cpu().numpy()
    keys = _score_keys(lay, lca, 1, HI, k)
    got = lay.download()
    flips = 0
    for r in (0, 13, 31):
        say("csa_decode_128k row", r)
        V = oracle.row_view(ref, r)
        oracle.compress_append(V, tok["kv"][r:r + 1], tok["gate"][r:r + 1], tok["ikey"][r:r + 1],
                               tok["igate"][r:r + 1])
        assert int(got["seq_len"][r]) == ctx
        slot = (ctx - 1) % V["ring"]
        assert np.array_equal(got["ring_kv"][r, slot], V["ring_kv"][0, slot])
        flips += _check_finalised(got, V, r, ctx // m - 1, m, True)
        sc = oracle.indexer_scores(V, 0, 0, 1, Q["iq"][r:r + 1], Q["iw"][r:r + 1])
        check_indexer_keys(*indexer_row_keys(*keys, r, len(sc)), sc, k)
        want = oracle.indexer_topk(V, Q["iq"][r:r + 1], Q["iw"][r:r + 1], k)
        check_topk(got_topk[r, 0], want[0, 0], sc, k)
        assert set(planted[r]) <= set(got_topk[r, 0].tolist())
        wo = oracle.csa_attend(V, Q["q"][r:r + 1], got_topk[r:r + 1], SCALE)
        err = attn_rel_err(got_out[r:r + 1], wo)
        print("row", r, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL
    assert flips <= 2


def test_hca_decode_1m_fullsize():
    """16 rows x 1048576 tokens (8192 entries), 64 heads, W = 128; the step
    finalises entry 8191 (a 128-token pooling)."""
    lca = _lca()
    B, ctx, m, H, W = 16, 1048576, 128, 64, 128
    seed, tag = 1002, "hca"
    say("hca_decode_1m fullsize B", B, "ctx", ctx, "seed", seed)
    ref = SL.make_layer(seed, tag, B, m, W, 256, 0, ctx // m + 64, [ctx - 1] * B)
    Q = SL.queries(seed, tag, B, 1, H)
    tok = SL.tokens(seed, "fullsize_step", B, 1, 0)
    lay = lca.Layer.from_host(ref)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]))
    out = lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
    torch.cuda.synchronize()
    got_out = out.cpu().numpy()
    got = lay.download()
    flips = 0
    for r in (0, 9, 15):
        say("hca_decode_1m row", r)
        V = oracle.row_view(ref, r)
        oracle.compress_append(V, tok["kv"][r:r + 1], tok["gate"][r:r + 1])
        assert int(got["seq_len"][r]) == ctx
        flips += _check_finalised(got, V, r, ctx // m - 1, m, False)
        wo = oracle.hca_attend(V, Q["q"][r:r + 1], SCALE)
        err = attn_rel_err(got_out[r:r + 1], wo)
        print("row", r, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL
    assert flips <= 2


def test_csa_prefill_chunk_fullsize():
    """One row with a 262144-token prior context (65536 blocks): a 4096-token
    chunk goes through compress_append (1024 new blocks), then 4096 queries
    select their causal top-512 among up to 66560 blocks and attend.  Sampled
    queries are checked against the oracle."""
    lca = _lca()
    prior, n, m, H, HI, k, W, R = 262144, 4096, 4, 64, 16, 512, 128, 8192
    seed, tag = 1004, "prefill"
    say("csa_prefill_chunk fullsize prior", prior, "chunk", n, "seed", seed)
    ref = SL.make_layer(seed, tag, 1, m, W, R, 1, (prior + n) // m + 64, [prior])
    tok = SL.tokens(seed, "chunk", 1, n, 1)
    Q = SL.queries(seed, tag, 1, n, H, HI)
    lay = lca.Layer.from_host(ref)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]), _dev(tok["ikey"]), _dev(tok["igate"]))
    topk = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
    out = lca.csa_attend(lay, _dev(Q["q"]), topk, float(SCALE))
    torch.cuda.synchronize()
    got_topk = topk.cpu().numpy()
    keys = _score_keys(lay, lca, n, HI, k)
    got = lay.download()
    V = oracle.row_view(ref, 0)
    oracle.compress_append(V, tok["kv"], tok["gate"], tok["ikey"], tok["igate"])
    assert int(got["seq_len"][0]) == prior + n
    flips = 0
    for b in (prior // m, prior // m + 511, (prior + n) // m - 1):
        flips += _check_finalised(got, V, 0, b, m, True)
    assert flips <= 2
    for qi in (0, 1, 1234, 4094, 4095):
        say("csa_prefill query", qi)
        sc = oracle.indexer_scores(V, 0, qi, n, Q["iq"], Q["iw"])
        check_indexer_keys(*indexer_row_keys(*keys, qi, len(sc)), sc, k)
        check_topk(got_topk[0, qi], oracle.topk_select(sc, k), sc, k)
        # one query alone: a view whose length ends at the query's position
        p = prior + qi
        Vq = dict(V)
        Vq["seq_len"] = np.array([p + 1], np.int32)
        wo = oracle.csa_attend(Vq, Q["q"][:, qi:qi + 1], got_topk[:, qi:qi + 1], SCALE)
        err = attn_rel_err(out[:, qi:qi + 1].cpu().numpy(), wo)
        print("query", qi, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL


def test_hca_prefill_chunk_fullsize():
    """One HCA row with a 262144-token prior context (2048 blocks at m = 128):
    a 4096-token chunk goes through compress_append (32 new blocks), then its
    4096 queries attend densely to the blocks each one sees, plus the window.
    Sampled queries (around block boundaries and at both ends) are checked
    against the oracle."""
    lca = _lca()
    prior, n, m, H, W, R = 262144, 4096, 128, 64, 128, 8192
    seed, tag = 1005, "hprefill"
    say("hca_prefill_chunk fullsize prior", prior, "chunk", n, "seed", seed)
    ref = SL.make_layer(seed, tag, 1, m, W, R, 0, (prior + n) // m + 64, [prior])
    tok = SL.tokens(seed, "chunk", 1, n, 0)
    Q = SL.queries(seed, tag, 1, n, H)
    lay = lca.Layer.from_host(ref)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]))
    out = lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
    torch.cuda.synchronize()
    got = lay.download()
    V = oracle.row_view(ref, 0)
    oracle.compress_append(V, tok["kv"], tok["gate"])
    assert int(got["seq_len"][0]) == prior + n
    flips = 0
    for b in (prior // m, (prior + n) // m - 1):
        flips += _check_finalised(got, V, 0, b, m, False)
    assert flips <= 2
    for qi in (0, 126, 127, 2047, 4095):
        say("hca_prefill query", qi)
        Vq = dict(V)
        Vq["seq_len"] = np.array([prior + qi + 1], np.int32)
        wo = oracle.hca_attend(Vq, Q["q"][:, qi:qi + 1], SCALE)
        err = attn_rel_err(out[:, qi:qi + 1].cpu().numpy(), wo)
        print("query", qi, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL


def _row_copy(L, r):
    """an independent one-row copy of row r of a layer image"""
    V = dict(L)
    V["batch"] = 1
    for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv", "ring_gate",
              "ring_ikey", "ring_igate"):
        V[f] = np.ascontiguousarray(L[f][r:r + 1]).copy()
    return V


def _device_row(lay, r):
    """row r of a device layer as a one-row host dict (the planes an entry check reads)"""
    out = {}
    for f in ("nope", "rope", "kv_scale", "idx_code", "idx_scale"):
        t = getattr(lay, f)
        if t is not None and t.numel():
            a = t[r:r + 1].cpu().numpy()
            out[f] = a.view(np.uint16) if a.dtype == np.int16 else a
    return out


def test_interleaved_1m_fullsize():
    """8 rows at a 1048575-token context, 8 CSA layers (16 heads, 4 indexer
    heads, k = 64) interleaved with 8 HCA layers (64 heads), 26 outlier
    channels x20; six decode steps (step 0 finalises CSA block 262143 and HCA
    entry 8191, step 4 finalises CSA block 262144).  Two sampled rows of the
    first CSA and the last HCA layer are followed by the oracle through every
    step and checked at the end."""
    lca = _lca()
    B, ctx, P, H_c, HI, k, H_h, W = 8, 1 << 20, 8, 16, 4, 64, 64, 128
    seed = 1005
    say("interleaved_1m fullsize B", B, "pairs", P, "seed", seed)
    images, ch = {}, {}
    for kind, m, has_idx in (("csa", 4, 1), ("hca", 128, 0)):
        ref = SL.make_layer(seed, kind, B, m, W, 256, has_idx, ctx // m + 64, [ctx - 1] * B)
        ch[kind] = SL.outlier_channels(seed, kind, 0)
        SL.apply_outliers(ref, ch[kind])
        images[kind] = ref
    layers = {kind: [lca.Layer.from_host(images[kind]) for _ in range(P)] for kind in ("csa", "hca")}
    rows = (2, 7)
    track = {("csa", 0): {r: _row_copy(images["csa"], r) for r in rows},
             ("hca", P - 1): {r: _row_copy(images["hca"], r) for r in rows}}
    del images
    steps = 6
    for s in range(steps):
        say("interleaved step", s)
        qc = SL.queries(seed, "csaq", B, 1, H_c, HI, step=s)
        qh = SL.queries(seed, "hcaq", B, 1, H_h, step=s)
        for l in range(P):
            tc = SL.outlier_tokens(SL.tokens(seed, f"csa{l}", B, 1, 1, step=s), ch["csa"])
            th = SL.outlier_tokens(SL.tokens(seed, f"hca{l}", B, 1, 0, step=s), ch["hca"])
            c, h = layers["csa"][l], layers["hca"][l]
            lca.compress_append(c, _dev(tc["kv"]), _dev(tc["gate"]), _dev(tc["ikey"]), _dev(tc["igate"]))
            topk = lca.indexer_topk(c, _dev(qc["iq"]), _dev(qc["iw"]), k)
            out_c = lca.csa_attend(c, _dev(qc["q"]), topk, float(SCALE))
            lca.compress_append(h, _dev(th["kv"]), _dev(th["gate"]))
            out_h = lca.hca_attend(h, _dev(qh["q"]), float(SCALE))
            for (kind, tl), views in track.items():
                if tl != l:
                    continue
                t = tc if kind == "csa" else th
                for r, V in views.items():
                    if kind == "csa":
                        oracle.compress_append(V, t["kv"][r:r + 1], t["gate"][r:r + 1], t["ikey"][r:r + 1],
                                               t["igate"][r:r + 1])
                    else:
                        oracle.compress_append(V, t["kv"][r:r + 1], t["gate"][r:r + 1])
            if l == 0:
                csa_topk, csa_out = topk, out_c
            if l == P - 1:
                hca_out = out_h
        torch.cuda.synchronize()
    got_topk, got_c, got_h = csa_topk.cpu().numpy(), csa_out.cpu().numpy(), hca_out.cpu().numpy()
    flips = 0
    for r, V in track[("csa", 0)].items():
        say("interleaved csa layer 0 row", r)
        dev_row = _device_row(layers["csa"][0], r)
        for b in (ctx // 4 - 1, ctx // 4):
            flips += _check_finalised(dev_row, V, 0, b, 4, True)
        want = oracle.indexer_topk(V, qc["iq"][r:r + 1], qc["iw"][r:r + 1], k)
        check_topk(got_topk[r, 0], want[0, 0],
                   oracle.indexer_scores(V, 0, 0, 1, qc["iq"][r:r + 1], qc["iw"][r:r + 1]), k)
        wo = oracle.csa_attend(V, qc["q"][r:r + 1], got_topk[r:r + 1], SCALE)
        err = attn_rel_err(got_c[r:r + 1], wo)
        print("csa row", r, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL
    for r, V in track[("hca", P - 1)].items():
        say("interleaved hca layer", P - 1, "row", r)
        dev_row = _device_row(layers["hca"][P - 1], r)
        flips += _check_finalised(dev_row, V, 0, ctx // 128 - 1, 128, False)
        wo = oracle.hca_attend(V, qh["q"][r:r + 1], SCALE)
        err = attn_rel_err(got_h[r:r + 1], wo)
        print("hca row", r, "attention max rel err", err, flush=True)
        assert err <= ATTN_TOL
    assert flips <= 4
