"""lca_indexer_topk_noalloc (static scratch array as workspace) against
lca_indexer_topk with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, then a larger one again, and a call
too large for the array, which fails before anything is enqueued."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth import layers as SL

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# (name, batch, lengths, n_q, H_I, k): the larger call first, then a smaller
# one (fewer rows, shorter, one query), then a chunk with more queries
CALLS = [("large", 2, [1048576, 600001], 2, 16, 512),
         ("small", 2, [9000, 4100], 1, 8, 64),
         ("chunk", 1, [30000], 24, 16, 256)]


def test_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_append_amd as lca
    for name, B, lens, n_q, H_I, k in CALLS:
        say("noalloc", name, "B", B, "lens", lens, "n_q", n_q, "H_I", H_I, "k", k)
        ref = SL.make_layer(95, name, B, 4, 128, 256, 1, max(lens) // 4 + 8, lens)
        Q = SL.queries(95, name, B, n_q, 16, H_I)
        Q["iw"] = SL.signed_weights(95, name, Q["iw"], "mixed")
        lay = lca.Layer.from_host(ref)
        iq, iw = _dev(Q["iq"]), _dev(Q["iw"])
        want = lca.indexer_topk(lay, iq, iw, k)
        got = lca.indexer_topk_noalloc(lay, iq, iw, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want), name
        again = lca.indexer_topk_noalloc(lay, iq, iw, k)
        torch.cuda.synchronize()
        assert torch.equal(again, want), name


def test_noalloc_rejects_a_call_beyond_the_array():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_append_amd as lca
    say("noalloc too large")
    B, L, n_q = 1, 60000, 512          # 512 queries x 15000 blocks of keys and lists
    lay = lca.Layer(B, 4, 128, 1024, True, L // 4 + 8, lengths=[L])
    need = lca.indexer_workspace_bytes(lay, n_q, 16, 64)
    assert need > (32 << 20)
    iq = torch.zeros((B, n_q, 16, 64), dtype=torch.float32, device="cuda")
    iw = torch.zeros((B, n_q, 16), dtype=torch.float32, device="cuda")
    out = torch.full((B, n_q, 64), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(lca.LcaError) as e:
        lca.indexer_topk_noalloc(lay, iq, iw, 64, out=out)
    assert e.value.code == -4
    torch.cuda.synchronize()
    assert bool((out == -7).all())      # nothing was enqueued
