"""The oracle on paged entry planes (a shared pool of pages and a per-row
page table, the library's layout for variable-length batches).

Paging is storage only: every result on a paged layer must equal, bit for
bit, the result on the contiguous layer holding the same entries.  These
tests pin the oracle's page lookup to that property (a wrong page, offset or
row in the lookup reads another entry, or one of the spare pool pages filled
with random codes, and changes a result), and check that an entry on an
unmapped page is an error.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import layers as SL

SCALE = np.float32(1.0 / np.sqrt(512.0))


def _layers(seed, csa, lengths, PB=64, reserve=24):
    m = 4 if csa else 16
    L = SL.make_layer(seed, "paged", len(lengths), m, 32, 64, int(csa), 1024, lengths)
    P = SL.paginate(L, seed, PB, reserve_blocks=reserve)
    return L, P


@pytest.mark.parametrize("csa", [1, 0], ids=["csa", "hca"])
def test_paged_compress_writes_the_mapped_entries(csa):
    lengths = [700, 1999, 61]                     # ragged rows
    L, P = _layers(31, csa, lengths)
    spare = np.ones(P["pool_pages"], bool)
    spare[P["page_table"][P["page_table"] >= 0]] = False
    before = {f: P[f].copy() for f in SL.ENTRY_PLANES}
    tok = SL.tokens(31, "paged", len(lengths), 40, csa)
    oracle.compress_append(L, tok["kv"], tok["gate"], tok.get("ikey"), tok.get("igate"))
    oracle.compress_append(P, tok["kv"], tok["gate"], tok.get("ikey"), tok.get("igate"))
    assert (P["seq_len"] == L["seq_len"]).all()
    U = SL.unpaginate(P)
    m = L["ratio"]
    for r, n0 in enumerate(lengths):
        nb = (n0 + 40) // m
        assert nb > n0 // m                        # the call finalised blocks in every row
        for f in SL.ENTRY_PLANES:
            if L[f].size:
                assert (U[f][r, :nb] == L[f][r, :nb]).all(), (f, r)
    PB = P["page_blocks"]
    for pg in np.nonzero(spare)[0]:                # pages no row maps are untouched
        for f in SL.ENTRY_PLANES:
            if P[f].size:
                assert (P[f][pg * PB:(pg + 1) * PB] == before[f][pg * PB:(pg + 1) * PB]).all()
    for f in ("ring_kv", "ring_gate"):
        assert (P[f] == L[f]).all()


def test_paged_indexer_equals_contiguous():
    lengths = [2001, 777, 4000]
    L, P = _layers(32, 1, lengths)
    Q = SL.queries(32, "paged", len(lengths), 3, 8, 8)
    for k in (16, 600):
        a = oracle.indexer_topk(L, Q["iq"], Q["iw"], k)
        b = oracle.indexer_topk(P, Q["iq"], Q["iw"], k)
        assert (a == b).all()
    for r in range(len(lengths)):
        sa = oracle.indexer_scores(L, r, 2, 3, Q["iq"], Q["iw"])
        sb = oracle.indexer_scores(P, r, 2, 3, Q["iq"], Q["iw"])
        assert sa.view(np.uint32).tolist() == sb.view(np.uint32).tolist()


@pytest.mark.parametrize("csa", [1, 0], ids=["csa", "hca"])
def test_paged_attend_equals_contiguous(csa):
    lengths = [1500, 333, 2600]
    L, P = _layers(33, csa, lengths)
    Q = SL.queries(33, "paged", len(lengths), 2, 4, 4)
    if csa:
        tk = oracle.indexer_topk(L, Q["iq"], Q["iw"], 48)
        a = oracle.csa_attend(L, Q["q"], tk, SCALE)
        b = oracle.csa_attend(P, Q["q"], tk, SCALE)
    else:
        a = oracle.hca_attend(L, Q["q"], SCALE)
        b = oracle.hca_attend(P, Q["q"], SCALE)
    assert a.view(np.uint32).tolist() == b.view(np.uint32).tolist()


def test_paged_lookup_places_entries_by_page_and_offset():
    """Entry b of row r sits at page_table[r][b // PB] * PB + b % PB, or
    nowhere (-1) on an unmapped page: checked on entries written with
    recognisable codes."""
    L, P = _layers(34, 1, [900, 300], PB=128, reserve=0)
    PB = P["page_blocks"]
    for r in range(2):
        for b in (0, 1, PB - 1, PB, 3 * PB + 5, 899 // 4):
            e = oracle.entry_index(P, r, b)
            pg = P["page_table"][r, b // PB]
            assert e == (-1 if pg < 0 else pg * PB + b % PB)
            if e >= 0 and b < int(P["seq_len"][r]) // 4:
                assert (P["nope"][e] == L["nope"][r, b]).all()
    assert oracle.entry_index(P, 1, 300 // 4 + PB) == -1


def test_unmapped_page_is_an_error():
    L, P = _layers(35, 1, [1000, 1000], reserve=0)
    tok = SL.tokens(35, "paged", 2, 64, 1)
    row_pages = P["page_table"][0]
    assert (row_pages[(1000 // 4) // 64 + 1:] == -1).all()
    with pytest.raises(RuntimeError, match=r"\(-8\)"):
        oracle.compress_append(P, tok["kv"], tok["gate"], tok["ikey"], tok["igate"])
    P2 = dict(P)
    P2["page_table"] = P["page_table"].copy()
    P2["page_table"][1, 0] = -1                     # a visible entry's page unmapped
    Q = SL.queries(35, "paged", 2, 1, 4, 4)
    with pytest.raises(RuntimeError, match=r"\(-8\)"):
        oracle.indexer_topk(P2, Q["iq"], Q["iw"], 8)
    with pytest.raises(RuntimeError, match=r"\(-8\)"):
        oracle.hca_attend(P2, Q["q"], SCALE)
