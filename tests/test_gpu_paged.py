"""GPU parity on paged entry planes: rows of a batch draw their compressed
entries from one pool of pages through a per-row page table (variable-length
batches).  Every call is checked against the oracle on the same paged layer
(the oracle's page lookup is pinned on the CPU to the contiguous results),
with the bars of the contiguous tests: entries equal up to rounding-midpoint
code flips, top-k sets under the 1e-6 tie rule, attention within 2e-3.
Pool pages no row maps hold random codes and must stay untouched; a read of
one of them would change a result."""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from synth import layers as SL

from gpu_helpers import ATTN_TOL, attn_rel_err, check_topk, compare_entries

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


def _spare_pages(P):
    used = np.zeros(P["pool_pages"], bool)
    used[P["page_table"][P["page_table"] >= 0]] = True
    return np.nonzero(~used)[0]


def _check_spares(got, before, P):
    PB = P["page_blocks"]
    for pg in _spare_pages(P):
        for f in SL.ENTRY_PLANES:
            if before[f].size:
                assert np.array_equal(got[f][pg * PB:(pg + 1) * PB], before[f][pg * PB:(pg + 1) * PB]), (f, pg)


# ------------------------------------------------------------------ compressor

PAGED_COMPRESS_CASES = [
    # (name, ratio, has_idx, window, ring, batch, initial lengths, appends, page_blocks)
    ("csa_m4_pb64", 4, 1, 16, 64, 3, [0, 700, 1501], [37, 1, 1, 1, 9, 3], 64),
    ("hca_m128_pb64", 128, 0, 16, 300, 2, [9000, 100], [130, 1, 60, 70], 64),
    ("m16_idx_pb128", 16, 1, 16, 64, 2, [2000, 7], [40, 1, 30, 9], 128),
]


@pytest.mark.parametrize("case", PAGED_COMPRESS_CASES, ids=[c[0] for c in PAGED_COMPRESS_CASES])
def test_paged_compress_append_parity(case):
    lca = _lca()
    name, m, hi, W, R, B, lens0, appends, PB = case
    seed = 5000 + zlib.crc32(name.encode()) % 1000
    say("paged compress", name, "m", m, "B", B, "lens", lens0, "appends", appends, "PB", PB, "seed", seed)
    total = max(lens0) + sum(appends)
    MB = ((total // m + 2) + PB - 1) // PB * PB
    hist = SL.tokens(seed, "hist", B, total, hi)
    base = SL.empty_layer(B, m, W, R, hi, MB)
    base["pos_bias"], base["ipos_bias"] = SL.pos_bias(seed, name, m, hi)
    for b in range(B):                            # initial rows, appended on the oracle side
        one = SL.empty_layer(1, m, W, R, hi, MB)
        one["pos_bias"], one["ipos_bias"] = base["pos_bias"], base["ipos_bias"]
        if lens0[b]:
            oracle.compress_append(one, hist["kv"][b:b + 1, :lens0[b]].copy(),
                                   hist["gate"][b:b + 1, :lens0[b]].copy(),
                                   hist["ikey"][b:b + 1, :lens0[b]].copy() if hi else None,
                                   hist["igate"][b:b + 1, :lens0[b]].copy() if hi else None)
        for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
                  "ring_gate", "ring_ikey", "ring_igate"):
            base[f][b] = one[f][0]
    ref = SL.paginate(base, seed, PB, reserve_blocks=sum(appends) // m + 1)
    before = {f: ref[f].copy() for f in SL.ENTRY_PLANES}
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
    assert lay.status() == 0
    got = lay.download()
    got["page_table"] = ref["page_table"]
    assert np.array_equal(got["seq_len"], ref["seq_len"])
    _check_spares(got, before, ref)
    gu, ru = SL.unpaginate(got), SL.unpaginate(ref)
    flips = 0
    for b in range(B):
        nb = int(pos[b]) // m
        t = np.arange(nb * m).reshape(nb, m)
        flips += compare_entries(gu, ru, b, list(range(nb)), hist["kv"][b][t], hist["gate"][b][t],
                                 hist["ikey"][b][t] if hi else None, hist["igate"][b][t] if hi else None,
                                 ref["pos_bias"], ref["ipos_bias"], m)
    n_codes = sum(int(p) // m for p in pos) * (448 + 64 + (64 if hi else 0))
    assert flips <= max(2, n_codes // 1000), flips


# ------------------------------------------------------------------ indexer

PAGED_INDEXER_CASES = [
    # (name, batch, lengths, n_q, H_I, k, page_blocks)
    ("decode_ragged_h16_k512_pb64", 4, [9000, 4100, 61000, 300], 1, 16, 512, 64),
    ("decode_long_h16_k512_pb4096", 2, [140000, 33000], 1, 16, 512, 4096),
    ("decode_h4_k64_pb256", 3, [4096, 20000, 777], 1, 4, 64, 256),
    ("chunk_nq64_h16_k256_pb128", 2, [30000, 20011], 64, 16, 256, 128),
    ("chunk_nq20_h32_k64_pb2048", 1, [50000], 20, 32, 64, 2048),
]
PAGED_INDEXER_MODES = {"auto": {}, "sliced": {"LCA_TOPK_SLICED": 1},
                       "separate": {"LCA_TOPK_FUSED": 0, "LCA_TOPK_SLICED": 0},
                       "tile_cand": {"LCA_SCORE_TILE": 1, "LCA_TOPK_CAND": 1},
                       "tile_full": {"LCA_SCORE_TILE": 1, "LCA_TOPK_CAND": 0}}
_ORACLE = {}


@pytest.mark.parametrize("mode", list(PAGED_INDEXER_MODES))
@pytest.mark.parametrize("case", PAGED_INDEXER_CASES, ids=[c[0] for c in PAGED_INDEXER_CASES])
def test_paged_indexer_topk_parity(case, mode, tuning):
    lca = _lca()
    name, B, lens, n_q, H_I, k, PB = case
    seed = 5200 + len(name)
    say("paged indexer", name, "B", B, "lens", lens, "n_q", n_q, "H_I", H_I, "k", k, "PB", PB, "mode", mode)
    for var, val in PAGED_INDEXER_MODES[mode].items():
        tuning(var, val)
    m = 4
    MB = (max(lens) // m + 8 + PB - 1) // PB * PB
    base = SL.make_layer(seed, name, B, m, 128, 256, 1, MB, lens)
    Q = SL.queries(seed, name, B, n_q, 16, H_I)
    Q["iw"] = SL.signed_weights(seed, name, Q["iw"], "mixed")
    ref = SL.paginate(base, seed, PB)
    lay = lca.Layer.from_host(ref)
    got = lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), k)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert lay.status() == 0
    if name not in _ORACLE:
        _ORACLE[name] = (oracle.indexer_topk(ref, Q["iq"], Q["iw"], k),
                         {(b, qi): oracle.indexer_scores(ref, b, qi, n_q, Q["iq"], Q["iw"])
                          for b in range(B) for qi in sorted({0, n_q // 2, n_q - 1})})
    want, scores = _ORACLE[name]
    for b in range(B):
        for qi in range(n_q):
            if (b, qi) in scores:
                check_topk(got[b, qi], want[b, qi], scores[(b, qi)], k)
            else:
                assert np.array_equal(got[b, qi], want[b, qi]), (b, qi)


# ------------------------------------------------------------------ attention

PAGED_ATTEND_CASES = [
    # (name, csa, batch, lengths, n_q, H, k, page_blocks)
    ("hca_ragged_h64_pb64", 0, 3, [200000, 9001, 300], 1, 64, 0, 64),
    ("csa_ragged_h64_k512_pb256", 1, 3, [90000, 6000, 2100], 1, 64, 512, 256),
    ("csa_chunk_nq40_h16_k64_pb64", 1, 2, [3000, 9000], 40, 16, 64, 64),
    ("hca_chunk_nq8_h16_pb128", 0, 1, [70000], 8, 16, 0, 128),
]


@pytest.mark.parametrize("case", PAGED_ATTEND_CASES, ids=[c[0] for c in PAGED_ATTEND_CASES])
def test_paged_attend_parity(case):
    lca = _lca()
    name, csa, B, lens, n_q, H, k, PB = case
    seed = 5400 + len(name)
    say("paged attend", name, "csa", csa, "B", B, "lens", lens, "n_q", n_q, "H", H, "k", k, "PB", PB)
    m, W = (4 if csa else 128), 128
    MB = (max(lens) // m + 8 + PB - 1) // PB * PB
    base = SL.make_layer(seed, name, B, m, W, max(256, n_q + W), csa, MB, lens)
    ref = SL.paginate(base, seed, PB)
    Q = SL.queries(seed, name, B, n_q, H, 4 if csa else 0)
    lay = lca.Layer.from_host(ref)
    if csa:
        rng = np.random.default_rng(seed)
        topk = np.full((B, n_q, k), -1, np.int32)
        for b in range(B):
            for qi in range(n_q):
                nv = (lens[b] - n_q + qi + 1) // m
                take = min(k - 1, nv)
                topk[b, qi, :take] = np.sort(rng.choice(nv, size=take, replace=False))
        want = oracle.csa_attend(ref, Q["q"], topk, SCALE)
        got = lca.csa_attend(lay, _dev(Q["q"]), _dev(topk), float(SCALE))
    else:
        want = oracle.hca_attend(ref, Q["q"], SCALE)
        got = lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
    torch.cuda.synchronize()
    err = attn_rel_err(got.cpu().numpy(), want)
    print("max rel err", err)
    assert err <= ATTN_TOL
    assert lay.status() == 0


# ------------------------------------------------------------------ unmapped pages

def test_unmapped_pages_are_reported():
    """A block to finalise on an unmapped page is not written; a visible
    block on an unmapped page is read by neither the indexer nor attention
    from outside the pool; each sets LCA_STATUS_PAGE."""
    lca = _lca()
    say("paged unmapped pages")
    B, L, PB = 2, 4096, 64
    base = SL.make_layer(5600, "unmapped", B, 4, 128, 256, 1, 1088, [L, L])
    ref = SL.paginate(base, 5600, PB, reserve_blocks=0)
    # 1024 blocks fill pages 0..15; appending 64 tokens completes blocks
    # 1024..1039, on page 16: unmapped
    assert (ref["page_table"][:, 16] == -1).all()
    lay = lca.Layer.from_host(ref)
    before = lay.download()
    tok = SL.tokens(5600, "unmapped", B, 64, 1)
    lca.compress_append(lay, _dev(tok["kv"]), _dev(tok["gate"]), _dev(tok["ikey"]), _dev(tok["igate"]))
    torch.cuda.synchronize()
    assert lay.status() == lca.STATUS_PAGE
    after = lay.download()
    for f in SL.ENTRY_PLANES:
        assert np.array_equal(after[f], before[f]), f
    # a visible entry's page unmapped: indexer and attention report it
    for call in ("indexer", "csa", "hca"):
        P = dict(ref)
        P["page_table"] = ref["page_table"].copy()
        P["page_table"][1, 3] = -1
        lay = lca.Layer.from_host(P)
        Q = SL.queries(5600, "unmapped", B, 1, 16, 4)
        if call == "indexer":
            lca.indexer_topk(lay, _dev(Q["iq"]), _dev(Q["iw"]), 64)
        elif call == "csa":
            topk = np.tile(np.arange(0, 640, 10, dtype=np.int32), (B, 1, 1))
            lca.csa_attend(lay, _dev(Q["q"]), _dev(topk), float(SCALE))
        else:
            lca.hca_attend(lay, _dev(Q["q"]), float(SCALE))
        torch.cuda.synchronize()
        assert lay.status() == lca.STATUS_PAGE, call


# ------------------------------------------------------------------ graph replay, no-allocation entry point

@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_paged_graph_replay_with_append(kind):
    """A paged layer's decode step (append, then selection and attention for
    CSA, or attention for HCA) captured once and replayed six times against
    an eager twin: top-k lists, outputs, lengths and the page pool agree bit
    for bit, across a finalised block (the table maps the pages to come)."""
    lca = _lca()
    csa = kind == "csa"
    B, H, HI, k, steps, PB = 3, 64, 16, 256, 6, 64
    m, lens = (4, [20001, 6003, 12999]) if csa else (128, [128 * 90 - 3, 128 * 40 - 1, 128 * 70 - 2])
    say("paged graph replay", kind, B, lens, steps, "PB", PB)
    MB = (max(lens) // m + 8 + PB - 1) // PB * PB
    base = SL.make_layer(5700, "pgr" + kind, B, m, 128, 256, int(csa), MB, lens)
    ref = SL.paginate(base, 5700, PB, reserve_blocks=steps // m + 2)
    tok = SL.tokens(5700, "pgr" + kind, B, 1, int(csa))
    Q = SL.queries(5700, "pgr" + kind, B, 1, H, HI if csa else 0)
    lg, le = lca.Layer.from_host(ref), lca.Layer.from_host(ref)
    d = {kk: _dev(v) for kk, v in tok.items()}
    q = _dev(Q["q"])
    iq, iw = (_dev(Q["iq"]), _dev(Q["iw"])) if csa else (None, None)
    bufs = {id(lay): (torch.empty((B, 1, k), dtype=torch.int32, device="cuda"),
                      torch.empty((B, 1, H, 512), dtype=torch.float32, device="cuda")) for lay in (lg, le)}

    def step(lay, plan_len=None):
        lca.compress_append(lay, d["kv"], d["gate"], d.get("ikey"), d.get("igate"))
        if plan_len is not None:
            lay.len_max = plan_len
        t, o = bufs[id(lay)]
        if csa:
            lca.indexer_topk(lay, iq, iw, k, out=t)
            lca.csa_attend(lay, q, t, float(SCALE), out=o)
        else:
            lca.hca_attend(lay, q, float(SCALE), out=o)

    final = max(lens) + steps + 2
    before = (lg.len_min, lg.len_max)
    lg.len_max = final
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
    lg.len_min, lg.len_max = before
    for r in range(steps):
        g.replay()
        step(le)
        torch.cuda.synchronize()
        (tg, og), (te, oe) = bufs[id(lg)], bufs[id(le)]
        assert torch.equal(lg.seq_len, le.seq_len), r
        assert not csa or torch.equal(tg, te), r
        assert torch.equal(og, oe), r
    a, b = lg.download(), le.download()
    for f in SL.ENTRY_PLANES + ("ring_kv",):
        if f in a:
            assert np.array_equal(a[f], b[f]), f
    assert lg.status() == 0 and le.status() == 0
    assert any(int(b["seq_len"][r]) // m > lens[r] // m for r in range(B))   # a block was finalised


def test_paged_noalloc_matches_workspace_call():
    """The no-allocation indexer entry point on a paged layer: the same
    selection as the call with a caller workspace, twice in a row."""
    lca = _lca()
    say("paged noalloc")
    B, lens, H_I, k, PB = 3, [70000, 9000, 33333], 16, 512, 128
    MB = (max(lens) // 4 + 8 + PB - 1) // PB * PB
    base = SL.make_layer(5800, "pna", B, 4, 128, 256, 1, MB, lens)
    ref = SL.paginate(base, 5800, PB)
    Q = SL.queries(5800, "pna", B, 1, 16, H_I)
    lay = lca.Layer.from_host(ref)
    iq, iw = _dev(Q["iq"]), _dev(Q["iw"])
    want = lca.indexer_topk(lay, iq, iw, k)
    for _ in range(2):
        got = lca.indexer_topk_noalloc(lay, iq, iw, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
    assert lay.status() == 0
