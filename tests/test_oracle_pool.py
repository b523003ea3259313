"""The pooled oracle (oracle/pool.py) splits rows, heads and batch rows over
worker processes and slices the per-head and per-batch inputs (slopes, bias
tables, document labels) to match; it must give the values of the plain
oracle call on the whole tensors for every mask and modification."""
import numpy as np
import pytest

from oracle import attention
from oracle.pool import attention_parallel, default_workers


def _inputs(B=2, H=4, Hkv=2, Sq=70, Skv=90, D=16, seed=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Sq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    return q, k, v


CASES = [
    dict(), dict(causal=True), dict(causal=True, window=9, q_offset=20),
    dict(doc=True, causal=True), dict(alibi=True, causal=True), dict(softcap=3.0),
    dict(relbias=5, causal=True, prefix=11, q_offset=20), dict(doc=True, alibi=True, window=30),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: ",".join(f"{k}={v}" for k, v in c.items()) or "dense")
def test_pool_equals_plain_oracle(case):
    q, k, v = _inputs()
    B, H, Sq, _ = q.shape
    Skv = k.shape[2]
    rng = np.random.default_rng(9)
    kw = dict(causal=case.get("causal", False), window=case.get("window"),
              softcap=case.get("softcap"), q_offset=case.get("q_offset", 0), prefix=case.get("prefix"))
    if case.get("doc"):
        n = max(Sq + kw["q_offset"], Skv)
        kw["doc_ids"] = np.sort(rng.integers(0, 4, (B, n)), axis=1)
    if case.get("alibi"):
        kw["alibi_slopes"] = rng.random(H)
    if "relbias" in case:
        kw["rel_bias"] = rng.standard_normal((H, 2 * case["relbias"] + 1))
    Oref, Lref = attention(q, k, v, 0.3, **kw)
    stats = {}
    O, L = attention_parallel(q, k, v, 0.3, workers=2, rows_per_task=32, stats=stats, **kw)
    assert stats["workers"] == 2 and stats["tasks"] == B * H * 3
    np.testing.assert_array_equal(np.isneginf(L), np.isneginf(Lref))
    fin = np.isfinite(Lref)
    assert np.abs(O - Oref).max() <= 1e-12
    assert np.abs(L[fin] - Lref[fin]).max() <= 1e-12


def test_pool_subsets_leave_the_rest_nan():
    q, k, v = _inputs(B=2, H=2, Hkv=1)
    O, L = attention_parallel(q, k, v, 0.5, workers=2, heads=[1], batches=[0])
    assert np.isnan(O[1]).all() and np.isnan(O[0, 0]).all() and np.isfinite(O[0, 1]).all()
    Oref, Lref = attention(q, k, v, 0.5, heads=[1])
    assert np.abs(O[0, 1] - Oref[0, 1]).max() <= 1e-12
    assert np.abs(L[0, 1] - Lref[0, 1]).max() <= 1e-12


def test_default_workers_bounded():
    assert 1 <= default_workers() <= 16
    assert default_workers(limit=1) == 1


def test_backward_slices_sum_to_plain_oracle():
    """Per-slice gradients summed over a group's query heads equal the plain
    oracle's dK and dV; dQ slices equal its dQ."""
    from oracle import attention_backward
    from oracle.pool import attention_backward_slices
    q, k, v = _inputs(B=2, H=4, Hkv=2, Sq=40, Skv=50)
    g = np.random.default_rng(5).standard_normal(q.shape)
    kw = dict(causal=True, alibi_slopes=np.array([0.5, 0.25, 0.1, 0.05]), q_offset=10)
    dQ, dK, dV = attention_backward(q, k, v, g, 0.3, **kw)
    res = attention_backward_slices(q, k, v, g, 0.3, [(b, h) for b in range(2) for h in range(4)],
                                    workers=2, **kw)
    for b in range(2):
        for kh in range(2):
            sk = sum(res[(b, h)][1] for h in (2 * kh, 2 * kh + 1))
            sv = sum(res[(b, h)][2] for h in (2 * kh, 2 * kh + 1))
            assert np.abs(sk - dK[b, kh]).max() <= 1e-12 and np.abs(sv - dV[b, kh]).max() <= 1e-12
        for h in range(4):
            assert np.abs(res[(b, h)][0] - dQ[b, h]).max() <= 1e-12
