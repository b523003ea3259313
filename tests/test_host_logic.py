"""Host-side logic that needs no GPU: the benchmark's FLOP accounting and the
seeded input generators."""
import numpy as np
import pytest
import torch

import bench
import oracle
from workload import (WORKLOADS, alibi_slopes, document_ids, document_lengths, draw_qkv,
                      make_inputs)


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(causal=True, window=100),
                                dict(window=90), dict(documents=True, causal=True, window=64),
                                dict(documents=True), dict(documents=True, window=40),
                                dict(causal=True, prefix=250), dict(causal=True, prefix=90, window=60),
                                dict(sq=200, q_offset=500, causal=True),
                                dict(sq=300, q_offset=123, causal=True, window=77, documents=True),
                                dict(sq=100, q_offset=600, causal=True, prefix=256)])
def test_admitted_pairs_match_counting(kw):
    wl = WORKLOADS["dense"].with_(B=2, H=1, Hkv=1, S=700, D=64, doc_len_range=(30, 250), **kw)
    inp = make_inputs(wl) if wl.documents else None
    doc = inp.doc_ids if inp is not None else None
    want = sum(oracle.pair_count(wl.Sq, wl.Skv, causal=wl.causal, window=wl.window or None,
                                 doc_row=None if doc is None else doc[b], q_offset=wl.q_offset,
                                 prefix=wl.prefix) for b in range(2))
    assert bench.admitted_pairs(wl, doc) == want


def test_config_pair_counts():
    c = WORKLOADS["causal_gqa"]
    assert bench.admitted_pairs(c, None) // c.B == 33_558_528
    assert bench.admitted_pairs(WORKLOADS["dense"], None) // 4 == 4096 * 4096
    assert bench.admitted_pairs(WORKLOADS["alibi_d64"], None) == 536_887_296
    # prefix-LM: S(S+1)/2 + P(P-1)/2 per row; prefill chunk: Sq * off + Sq(Sq+1)/2
    p = WORKLOADS["prefix_lm"]
    assert bench.admitted_pairs(p, None) // p.B == 8192 * 8193 // 2 + 2048 * 2047 // 2
    c = WORKLOADS["chunked_prefill"]
    assert bench.admitted_pairs(c, None) == 4096 * 28672 + 4096 * 4097 // 2


def test_document_lengths_cover_and_range():
    for seed in range(5):
        lens = document_lengths(16384, seed)
        assert sum(lens) == 16384
        assert all(512 <= L <= 4096 for L in lens[:-1]) and 1 <= lens[-1] <= 4096
    ids = document_ids([3, 1, 2])
    assert ids.tolist() == [0, 0, 0, 1, 2, 2] and ids.dtype == np.int32


def test_alibi_slopes_geometric():
    s = alibi_slopes(8)
    assert s.dtype == np.float32 and np.allclose(s, 2.0 ** (-np.arange(1, 9)))


def test_draw_order_and_determinism():
    q, k, v = draw_qkv(1, 2, 1, 5, 6, 4, seed=3)
    g = torch.Generator().manual_seed(3)
    assert torch.equal(q, torch.randn((1, 2, 5, 4), generator=g))
    assert torch.equal(k, torch.randn((1, 1, 6, 4), generator=g))
    q2, _, _ = draw_qkv(1, 2, 1, 5, 6, 4, seed=3)
    assert torch.equal(q, q2)


def test_pair_lists_from_tile_classes():
    """The expected-list helper of the GPU block-mask tests, checked on causal
    classes: 256-row tile p holds key tiles 0..2p+1; tile 2p is partial for
    half 0 and full for half 1, tile 2p+1 is empty for half 0 and partial for
    half 1; all earlier tiles are full for both halves."""
    from oracle import tile_classes
    from tests._parity import pair_lists
    n = 6
    lists = pair_lists(tile_classes(n * 128, n * 128, 128, causal=True))
    assert len(lists) == n // 2
    for p, lst in enumerate(lists):
        want = [(j << 4) | 0xF for j in range(2 * p)] + [((2 * p) << 4) | 0xD, ((2 * p + 1) << 4) | 0x4]
        assert lst == want, p
    # an odd number of 128-row tiles: the last 256-row tile has no second half
    lists = pair_lists(tile_classes(3 * 128, 3 * 128, 128))
    assert lists[1] == [(j << 4) | 0x3 for j in range(3)]


def test_check_pair_lists_contract():
    """The block-mask checker accepts exactly the oracle's lists and rejects
    a wrong class, a listed empty half, a missing tile and a wrong order."""
    import numpy as np
    import pytest
    from oracle import tile_classes
    from tests._parity import check_pair_lists, pair_lists
    S = 512
    doc = np.repeat(np.arange(4), 128).astype(np.int32)          # one document per 128 positions
    doc[100:140] = 7                                              # a short document across a tile edge
    ref = tile_classes(S, S, 128, causal=True, doc_row=doc)
    lists = pair_lists(ref)
    nk = ref.shape[1]
    counts = np.array([len(x) for x in lists])
    arr = np.zeros((len(lists), nk), dtype=np.int64)
    for i, x in enumerate(lists):
        arr[i, :len(x)] = x
    check_pair_lists(counts, arr, ref)
    bad = arr.copy()
    bad[0, 0] |= 0x3 << 2                                         # a corrupted full flag
    with pytest.raises(AssertionError):
        check_pair_lists(counts, bad, ref)
    # half 1 of query tile 0 (rows 128-255, labels {1, 7}) against key tile 0
    # (labels {0, 7}): rows 128-139 (label 7) see keys 100-127 (label 7), so
    # the oracle finds it partial; against key tile 1 it is partial too. A
    # half the oracle finds empty must not be listed.
    assert ref[3, 0] == 0                                         # rows 384-511 vs keys 0-127: empty
    bad = arr.copy()
    entries = [int(e) for e in bad[1, :counts[1]]]
    assert all(e >> 4 != 0 for e in entries)
    bad[1, :counts[1] + 1] = [(0 << 4) | 0x4] + entries           # list key tile 0 for half 1 of tile 1
    with pytest.raises(AssertionError):
        check_pair_lists(counts + np.array([0, 1]), bad, ref)
    bad = arr.copy()                                              # one tile dropped
    with pytest.raises(AssertionError):
        check_pair_lists(counts - np.array([0, 1]), bad, ref)
    bad = arr.copy()                                              # two entries swapped
    bad[1, [0, 1]] = bad[1, [1, 0]]
    with pytest.raises(AssertionError):
        check_pair_lists(counts, bad, ref)
