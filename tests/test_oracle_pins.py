"""Pins of the CPU oracle to facts it does not compute itself.

Each test checks the oracle against something fixed by the pages or by
mathematics: worked examples whose answers follow by hand, closed forms,
invariants, a scalar brute force, and a library routine. The choices are such
that a plausible slip in the oracle (a dropped scale or normaliser, a wrong
sign or offset in a mask or an ALiBi bias, swapped K and V, a wrong grouped-head
map, LSE in the wrong log base) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import admitted, attention, pair_count
from tests._brute import brute_attention
from workload import alibi_slopes, document_ids, document_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------- the pages' own figures
def test_dense_pair_count_is_quadratic_as_printed():
    """Dense attention compares every token with every other one: 1,000 tokens
    make 1 million comparisons and doubling the length quadruples the work."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "quadratic_pairs.txt"))
            if l.strip() and not l.startswith("#")]
    table = {int(a): int(b) for a, b in rows}
    assert pair_count(1000, 1000) == table[1000]
    assert pair_count(2000, 2000) == table[2000] == 4 * table[1000]
    # 100,000 tokens -> 10 billion: counted on a band of rows and extrapolated
    # by the row-independence of the dense mask (each row admits every key).
    band = pair_count(10, 100_000)
    assert band * 10_000 == table[100_000]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["cases"],
                         ids=lambda c: c["name"])
def test_worked_examples(case):
    O, L = attention(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]), case["scale"],
                     causal=case.get("causal", False),
                     doc_ids=np.array(case["doc_ids"]) if "doc_ids" in case else None,
                     alibi_slopes=case.get("alibi_slopes"), softcap=case.get("softcap"))
    np.testing.assert_allclose(O, np.array(case["O"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(case["LSE"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------- closed forms
VARIANTS = [
    dict(),
    dict(causal=True),
    dict(causal=True, window=5),
    dict(window=3),
    dict(causal=True, alibi_slopes=[0.5, 0.25]),
    dict(softcap=2.0),
    dict(causal=True, softcap=3.0),
]


@pytest.mark.parametrize("kw", VARIANTS, ids=str)
def test_rows_sum_to_one(kw):
    """Softmax weights of every row sum to 1: with V = 1 every output is 1."""
    B, H, S, D = 1, 2, 23, 8
    q, k = rnd((B, H, S, D), 1), rnd((B, H, S, D), 2)
    v = np.ones((B, H, S, D))
    O, L = attention(q, k, v, 1 / math.sqrt(D), **kw)
    assert np.abs(O - 1).max() < TOL
    assert np.isfinite(L).all()


def test_equal_scores_give_mean_of_v_dense_and_causal():
    B, H, S, D = 2, 2, 17, 4
    q = np.zeros((B, H, S, D))
    k, v = rnd((B, H, S, D), 3), rnd((B, H, S, D), 4)
    O, L = attention(q, k, v, 0.7)
    assert np.abs(O - v.mean(axis=2, keepdims=True)).max() < TOL
    assert np.abs(L - math.log(S)).max() < TOL
    O, L = attention(q, k, v, 0.7, causal=True)
    counts = np.arange(1, S + 1)
    prefix_mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
    assert np.abs(O - prefix_mean).max() < TOL
    assert np.abs(L - np.log(counts)[None, None, :]).max() < TOL
    # K is irrelevant here; swapping K and V must change the answer.
    O2, _ = attention(q, v, k, 0.7)
    assert np.abs(O2 - v.mean(axis=2, keepdims=True)).max() > 1e-3


def test_single_admitted_key_returns_that_row():
    """Causal AND window 1 admits only the key at the query's own position:
    O = V[q] and LSE = that single scaled score."""
    B, H, S, D = 1, 3, 19, 8
    q, k, v = rnd((B, H, S, D), 5), rnd((B, H, S, D), 6), rnd((B, H, S, D), 7)
    scale = 0.3
    O, L = attention(q, k, v, scale, causal=True, window=1)
    assert np.abs(O - v).max() < TOL
    diag = np.einsum("bhsd,bhsd->bhs", q, k) * scale
    assert np.abs(L - diag).max() < TOL


def test_causal_row_zero_is_v0():
    B, H, S, D = 2, 2, 9, 4
    q, k, v = rnd((B, H, S, D), 8), rnd((B, H, S, D), 9), rnd((B, H, S, D), 10)
    O, L = attention(q, k, v, 0.5, causal=True)
    assert np.abs(O[:, :, 0] - v[:, :, 0]).max() < TOL
    assert np.abs(L[:, :, 0] - 0.5 * (q[:, :, 0] * k[:, :, 0]).sum(-1)).max() < TOL


def test_alibi_geometric_closed_form():
    """Q = 0 under causal ALiBi: row q weights key q - t by r^t, r = e^-slope,
    so the normaliser is the geometric sum (1 - r^(q+1)) / (1 - r)."""
    B, H, S, D = 1, 4, 33, 3
    slopes = alibi_slopes(H).astype(np.float64)
    q = np.zeros((B, H, S, D))
    k, v = rnd((B, H, S, D), 11), rnd((B, H, S, D), 12)
    O, L = attention(q, k, v, 1.0, causal=True, alibi_slopes=slopes)
    for h in range(H):
        r = math.exp(-slopes[h])
        for i in range(S):
            norm = (1 - r ** (i + 1)) / (1 - r)
            assert abs(L[0, h, i] - math.log(norm)) < TOL
            num = sum(r ** t * v[0, h, i - t] for t in range(i + 1))
            assert np.abs(O[0, h, i] - num / norm).max() < TOL


def test_softcap_limits_and_bound():
    B, H, S, D = 1, 2, 21, 8
    q, k, v = rnd((B, H, S, D), 13) * 3, rnd((B, H, S, D), 14) * 3, rnd((B, H, S, D), 15)
    # all-zero scores are fixed points of c*tanh(s/c)
    z = np.zeros_like(q)
    a = attention(z, k, v, 1.0, causal=True, softcap=5.0)
    b = attention(z, k, v, 1.0, causal=True)
    assert max(np.abs(a[0] - b[0]).max(), np.abs(a[1] - b[1]).max()) < TOL
    # a huge cap changes scores by ~ s^3 / (3 c^2), far below rounding
    a = attention(q, k, v, 0.35, softcap=1e8)
    b = attention(q, k, v, 0.35)
    assert max(np.abs(a[0] - b[0]).max(), np.abs(a[1] - b[1]).max()) < 1e-11
    # a small cap bounds every modified score by c, so LSE <= c + ln(count)
    c = 0.5
    _, L = attention(q, k, v, 1.0, softcap=c)
    assert (L <= c + math.log(S) + TOL).all()
    _, Lplain = attention(q, k, v, 1.0)
    assert (Lplain > c + math.log(S)).any()   # the cap is active on these inputs


# --------------------------------------------------------------- invariants
def test_constant_shift_moves_lse_only():
    """Adding c to every score of a row leaves O unchanged and adds c to LSE.
    A constant extra dimension (q_last = 1, k_last = c / scale) does exactly
    that."""
    B, H, S, D = 1, 2, 15, 6
    q, k, v = rnd((B, H, S, D), 16), rnd((B, H, S, D), 17), rnd((B, H, S, D), 18)
    scale, c = 0.4, 2.5
    q2 = np.concatenate([q, np.ones((B, H, S, 1))], axis=-1)
    k2 = np.concatenate([k, np.full((B, H, S, 1), c / scale)], axis=-1)
    v2 = np.concatenate([v, np.zeros((B, H, S, 1))], axis=-1)
    for kw in (dict(), dict(causal=True), dict(causal=True, window=4)):
        O1, L1 = attention(q, k, v, scale, **kw)
        O2, L2 = attention(q2, k2, v2, scale, **kw)
        assert np.abs(O1 - O2[..., :D]).max() < 1e-12
        assert np.abs(L2 - L1 - c).max() < 1e-12


def test_key_permutation_dense():
    B, H, S, D = 1, 2, 25, 4
    q, k, v = rnd((B, H, S, D), 19), rnd((B, H, S, D), 20), rnd((B, H, S, D), 21)
    perm = np.random.default_rng(0).permutation(S)
    O1, L1 = attention(q, k, v, 0.5)
    O2, L2 = attention(q, k[:, :, perm], v[:, :, perm], 0.5)
    assert np.abs(O1 - O2).max() < TOL and np.abs(L1 - L2).max() < TOL


def test_linear_in_v():
    B, H, S, D = 1, 2, 13, 4
    q, k = rnd((B, H, S, D), 22), rnd((B, H, S, D), 23)
    v1, v2 = rnd((B, H, S, D), 24), rnd((B, H, S, D), 25)
    a = attention(q, k, v1, 0.5, causal=True)[0]
    b = attention(q, k, v2, 0.5, causal=True)[0]
    c = attention(q, k, 2 * v1 - 3 * v2, 0.5, causal=True)[0]
    assert np.abs(c - (2 * a - 3 * b)).max() < 1e-11


def test_split_kv_merge():
    """Attention over keys [0, n) and [n, N) merges into attention over [0, N)
    through the two LSEs."""
    B, H, S, D, n = 1, 2, 31, 8, 12
    q, k, v = rnd((B, H, S, D), 26), rnd((B, H, S, D), 27), rnd((B, H, S, D), 28)
    O, L = attention(q, k, v, 0.35)
    O1, L1 = attention(q, k[:, :, :n], v[:, :, :n], 0.35)
    O2, L2 = attention(q, k[:, :, n:], v[:, :, n:], 0.35)
    Lm = np.logaddexp(L1, L2)
    Om = (np.exp(L1 - Lm)[..., None] * O1 + np.exp(L2 - Lm)[..., None] * O2)
    assert np.abs(Lm - L).max() < TOL and np.abs(Om - O).max() < TOL


def test_grouped_heads_equal_repeated_kv():
    """GQA: query heads 2g and 2g+1 read K/V head g (consecutive grouping)."""
    B, H, Hkv, S, D = 2, 6, 3, 14, 4
    q, k, v = rnd((B, H, S, D), 29), rnd((B, Hkv, S, D), 30), rnd((B, Hkv, S, D), 31)
    O1, L1 = attention(q, k, v, 0.5, causal=True)
    rep = H // Hkv
    O2, L2 = attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), 0.5, causal=True)
    assert np.abs(O1 - O2).max() == 0 and np.abs(L1 - L2).max() == 0
    # the strided map h % Hkv is a different answer
    idx = [h % Hkv for h in range(H)]
    O3, _ = attention(q, k[:, idx], v[:, idx], 0.5, causal=True)
    assert np.abs(O3 - O1).max() > 1e-3


def test_fully_masked_rows_are_zero_and_minus_inf():
    """Queries past the end of the keys whose document has no key: O = 0,
    LSE = -inf, and no NaN anywhere."""
    B, H, Sq, Skv, D = 1, 2, 12, 6, 4
    q, k, v = rnd((B, H, Sq, D), 32), rnd((B, H, Skv, D), 33), rnd((B, H, Skv, D), 34)
    doc = np.array([[0] * 4 + [1] * 4 + [2] * 4])
    O, L = attention(q, k, v, 0.5, causal=True, doc_ids=doc)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    empty = np.arange(Sq) >= 8          # document 2 starts at position 8 >= Skv
    assert (O[:, :, empty] == 0).all() and np.isneginf(L[:, :, empty]).all()
    assert np.isfinite(L[:, :, ~empty]).all()


# --------------------------------------------------------------- brute force
BRUTE = [
    dict(),
    dict(causal=True),
    dict(causal=True, window=4),
    dict(window=2),
    dict(docs=True),
    dict(docs=True, causal=True, window=3),
    dict(causal=True, alibi=True),
    dict(alibi=True),
    dict(softcap=1.5),
    dict(causal=True, softcap=4.0, docs=True),
    dict(causal=True, q_offset=3),
    dict(causal=True, window=4, alibi=True, q_offset=2),
    dict(docs=True, causal=True, q_offset=1, softcap=2.0),
    dict(causal=True, prefix=4),
    dict(causal=True, prefix=3, window=5, q_offset=2),
    dict(relbias=3),
    dict(causal=True, relbias=1, q_offset=2),
    dict(docs=True, window=4, relbias=6),
]


@pytest.mark.parametrize("kw", BRUTE, ids=str)
@pytest.mark.parametrize("shape", [(1, 2, 2, 9, 9, 4), (2, 4, 2, 11, 11, 3), (1, 2, 1, 7, 12, 5),
                                   (1, 2, 2, 13, 6, 2)])
def test_matches_scalar_brute_force(kw, shape):
    B, H, Hkv, Sq, Skv, D = shape
    q, k, v = rnd((B, H, Sq, D), 35), rnd((B, Hkv, Skv, D), 36), rnd((B, Hkv, Skv, D), 37)
    doc = None
    off = kw.get("q_offset", 0)
    if kw.get("docs"):
        n = max(Sq + off, Skv)
        doc = np.stack([document_ids(document_lengths(n, 40 + b, 2, 5)) for b in range(B)])
    slopes = alibi_slopes(H).astype(np.float64) if kw.get("alibi") else None
    args = dict(causal=kw.get("causal", False), window=kw.get("window"), doc_ids=doc,
                alibi_slopes=slopes, softcap=kw.get("softcap"), q_offset=off,
                prefix=kw.get("prefix"),
                rel_bias=rnd((H, 2 * kw["relbias"] + 1), 41) if "relbias" in kw else None)
    O, L = attention(q, k, v, 0.6, **args)
    Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.6,
                             **{a: (b.tolist() if isinstance(b, np.ndarray) else b)
                                for a, b in args.items()})
    Ob, Lb = np.array(Ob), np.array(Lb)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    assert np.abs(L[fin] - Lb[fin]).max(initial=0) < TOL
    assert np.abs(O - Ob).max() < TOL


# --------------------------------------------------------------- library routine
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    B, H, S, D = 2, 3, 40, 16
    q, k, v = rnd((B, H, S, D), 38), rnd((B, H, S, D), 39), rnd((B, H, S, D), 40)
    O, _ = attention(q, k, v, 0.2, causal=causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.2)
    assert np.abs(O - ref.numpy()).max() < 1e-12


# --------------------------------------------------------------- query offset and prefix-LM
def sdpa_masked(q, k, v, scale, mask):
    """torch's float64 attention with an explicit boolean mask [Sq, Skv]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def test_decode_step_sees_every_key():
    """One query at the last position of a causal sequence attends to all keys:
    plain (maskless) attention of that query."""
    B, H, Skv, D = 2, 3, 37, 8
    q, k, v = rnd((B, H, 1, D), 60), rnd((B, H, Skv, D), 61), rnd((B, H, Skv, D), 62)
    O, L = attention(q, k, v, 0.3, causal=True, q_offset=Skv - 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.3).numpy()
    assert np.abs(O - ref).max() < 1e-12
    s = np.einsum("bhd,bhjd->bhj", q[:, :, 0], k) * 0.3
    assert np.abs(L[:, :, 0] - np.log(np.exp(s).sum(-1))).max() < 1e-12


def test_chunked_prefill_is_bottom_right_causal():
    """Sq new queries after Skv - Sq cached keys: the causal mask is the lower
    triangle shifted right by Skv - Sq (torch.tril with that diagonal)."""
    Sq, Skv, D = 9, 23, 6
    q, k, v = rnd((1, 2, Sq, D), 63), rnd((1, 2, Skv, D), 64), rnd((1, 2, Skv, D), 65)
    O, _ = attention(q, k, v, 0.5, causal=True, q_offset=Skv - Sq)
    mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq).numpy()
    assert np.abs(O - sdpa_masked(q, k, v, 0.5, mask)).max() < 1e-12


def test_offset_rows_equal_rows_of_the_full_problem():
    """Queries Skv-Sq..Skv-1 of a square problem, given as a chunk with their
    offset, get the same rows (all variants that read positions)."""
    Skv, Sq, D, H = 20, 7, 4, 4
    q, k, v = rnd((1, H, Skv, D), 66), rnd((1, 2, Skv, D), 67), rnd((1, 2, Skv, D), 68)
    doc = document_ids(document_lengths(Skv, 9, 3, 8))[None]
    kw = dict(causal=True, window=6, doc_ids=doc, alibi_slopes=alibi_slopes(H).astype(np.float64))
    Of, Lf = attention(q, k, v, 0.4, **kw)
    Oc, Lc = attention(q[:, :, Skv - Sq:], k, v, 0.4, q_offset=Skv - Sq, **kw)
    assert np.abs(Oc - Of[:, :, Skv - Sq:]).max() < 1e-12
    assert np.abs(Lc - Lf[:, :, Skv - Sq:]).max() < 1e-12


def test_prefix_lm_closed_forms():
    S, D = 18, 5
    q, k, v = rnd((1, 2, S, D), 69), rnd((1, 2, S, D), 70), rnd((1, 2, S, D), 71)
    # a prefix covering every key is no mask at all; a prefix of 0 is causal
    Od, _ = attention(q, k, v, 0.7)
    assert np.abs(attention(q, k, v, 0.7, causal=True, prefix=S)[0] - Od).max() < 1e-12
    Oc, _ = attention(q, k, v, 0.7, causal=True)
    assert np.abs(attention(q, k, v, 0.7, causal=True, prefix=0)[0] - Oc).max() < 1e-12
    # a prefix P: full block on the first P keys, causal after (explicit mask)
    P = 7
    mask = torch.ones(S, S, dtype=torch.bool).tril().numpy()
    mask[:, :P] = True
    assert np.abs(attention(q, k, v, 0.7, causal=True, prefix=P)[0]
                  - sdpa_masked(q, k, v, 0.7, mask)).max() < 1e-12


def test_relative_bias_linear_table_is_alibi():
    """A table linear in the clipped distance, with R covering every distance,
    is ALiBi with that slope (exact)."""
    B, H, Sq, Skv, D, off = 1, 4, 11, 19, 5, 8
    q, k, v = rnd((B, H, Sq, D), 72), rnd((B, 2, Skv, D), 73), rnd((B, 2, Skv, D), 74)
    slopes = alibi_slopes(H).astype(np.float64)
    R = Sq + Skv + off
    table = slopes[:, None] * np.arange(-R, R + 1)[None, :]
    for causal in (False, True):
        Oa, La = attention(q, k, v, 0.4, causal=causal, q_offset=off, alibi_slopes=slopes)
        Or, Lr = attention(q, k, v, 0.4, causal=causal, q_offset=off, rel_bias=table)
        assert np.abs(Oa - Or).max() < 1e-12 and np.abs(La - Lr).max() < 1e-12


def test_relative_bias_clipping_and_constant_table():
    """A constant table moves LSE by the constant only; with R = 0 every pair
    takes the single entry; beyond R the end entries apply."""
    S, D = 9, 4
    q, k, v = rnd((1, 2, S, D), 75), rnd((1, 2, S, D), 76), rnd((1, 2, S, D), 77)
    O0, L0 = attention(q, k, v, 0.5, causal=True)
    Oc, Lc = attention(q, k, v, 0.5, causal=True, rel_bias=np.full((2, 7), 1.25))
    assert np.abs(O0 - Oc).max() < 1e-12 and np.abs(Lc - L0 - 1.25).max() < 1e-12
    O1, L1 = attention(q, k, v, 0.5, causal=True, rel_bias=np.array([[0.5], [-2.0]]))
    assert np.abs(O1 - O0).max() < 1e-12
    assert np.abs(L1[0, 0] - L0[0, 0] - 0.5).max() < 1e-12 and np.abs(L1[0, 1] - L0[0, 1] + 2.0).max() < 1e-12
    # R = 1 under causal: key == query gets entry 1, every earlier key entry 0
    tab = np.array([[0.0, 3.0, 7.0], [0.0, 3.0, 7.0]])
    _, Lr = attention(q, k, v, 0.5, causal=True, rel_bias=tab)
    s = np.einsum("hd,hjd->hj", q[0, :, 4], k[0]) * 0.5
    manual = np.log(np.exp(s[:, :4]).sum(-1) + np.exp(s[:, 4] + 3.0))
    assert np.abs(Lr[0, :, 4] - manual).max() < 1e-12


def test_offset_and_prefix_pair_counts():
    # Sq queries after `off` cached keys, causal: query i sees off + i + 1 keys
    Sq, off = 300, 500
    assert pair_count(Sq, Sq + off, causal=True, q_offset=off) == Sq * off + Sq * (Sq + 1) // 2
    # prefix P adds P(P - 1) / 2 pairs to causal (query q < P gains P - 1 - q keys)
    S, P = 400, 130
    assert pair_count(S, S, causal=True, prefix=P) == S * (S + 1) // 2 + P * (P - 1) // 2


# --------------------------------------------------------------- mask and pair-count closed forms
def window_doc_pairs(lengths, W):
    """Closed form: a document of length L under causal AND window W admits
    L(L+1)/2 pairs when L <= W, else W(W+1)/2 + (L - W) W."""
    tot = 0
    for L in lengths:
        tot += L * (L + 1) // 2 if L <= W else W * (W + 1) // 2 + (L - W) * W
    return tot


def test_pair_count_closed_forms():
    assert pair_count(300, 300, causal=True) == 300 * 301 // 2
    assert pair_count(257, 257) == 257 * 257
    lens = document_lengths(3000, 7, 100, 900)
    doc = document_ids(lens)
    assert pair_count(3000, 3000, causal=True, window=256, doc_row=doc) == window_doc_pairs(lens, 256)
    # window >= S is plain causal; one document is no document mask
    assert pair_count(200, 200, causal=True, window=200) == 200 * 201 // 2
    one = np.zeros(150, dtype=np.int32)
    assert pair_count(150, 150, doc_row=one) == 150 * 150


def test_mask_predicates_literal():
    qi, ki = np.arange(6)[:, None], np.arange(6)[None, :]
    assert admitted(qi, ki, causal=True).sum() == 21
    w = admitted(qi, ki, causal=True, window=2)
    assert w[3].tolist() == [False, False, True, True, False, False]   # keys 2 and 3


# --------------------------------------------------------------- tile classification
def test_tile_classes_causal_closed_form():
    """Causal, S = n tiles exactly: the diagonal tiles are partial, the n(n-1)/2
    below it full, the rest empty."""
    from oracle import tile_classes
    n, T = 6, 16
    c = tile_classes(n * T, n * T, T, causal=True)
    assert (np.diag(c) == 1).all()
    assert (c[np.tril_indices(n, -1)] == 2).all() and (c[np.triu_indices(n, 1)] == 0).all()
    assert (c == 2).sum() == n * (n - 1) // 2


def test_tile_classes_tails_and_window():
    from oracle import tile_classes
    # ragged keys: the last key tile is never full
    c = tile_classes(40, 40, 16)
    assert c.shape == (3, 3) and (c[:, :2] == 2).all() and (c[:, 2] == 1).all()
    # causal window of one tile width: two bands of partial tiles, nothing full
    c = tile_classes(64, 64, 16, causal=True, window=16)
    for i in range(4):
        for j in range(4):
            assert c[i, j] == (1 if j in (i - 1, i) else 0)
    # documents aligned to tiles: block-diagonal full tiles
    doc = np.repeat([0, 1], 32)
    c = tile_classes(64, 64, 16, doc_row=doc)
    assert (c == np.kron(np.eye(2, dtype=int), np.full((2, 2), 2))).all()
