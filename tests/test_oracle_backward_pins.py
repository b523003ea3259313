"""Pins of the oracle's gradients (CPU only): central finite differences of
the forward oracle, PyTorch float64 autograd, and identities the exact
derivative must satisfy. None of them re-types the gradient formulas."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

VARIANTS = [
    dict(),
    dict(causal=True),
    dict(causal=True, window=3),
    dict(window=2),
    dict(doc=True),
    dict(causal=True, doc=True),
    dict(alibi=True, causal=True),
    dict(softcap=2.0),
    dict(softcap=2.0, causal=True, window=4),
    dict(causal=True, prefix=3),
    dict(causal=True, q_offset=-2, alibi=True),
    dict(causal=True, doc=True, q_offset=2, window=5),
    dict(relbias=2),
    dict(relbias=1, causal=True, q_offset=1),
]


def _inputs(seed, B=1, H=2, Hkv=1, S=6, D=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    g = rng.standard_normal((B, H, S, D))
    return q, k, v, g


def _kw(var, S, H):
    kw = dict(causal=var.get("causal", False), window=var.get("window"),
              q_offset=var.get("q_offset", 0), prefix=var.get("prefix"))
    if var.get("doc"):
        kw["doc_ids"] = np.array([[0, 0, 0, 1, 1, 2, 2, 2][:S + max(0, kw["q_offset"])]])
    if var.get("alibi"):
        kw["alibi_slopes"] = np.array([0.5, 0.25][:H])
    if "softcap" in var:
        kw["softcap"] = var["softcap"]
    if "relbias" in var:
        kw["rel_bias"] = np.random.default_rng(9).standard_normal((H, 2 * var["relbias"] + 1))
    return kw


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: ",".join(f"{a}={b}" for a, b in v.items()) or "dense")
def test_gradients_match_central_differences(var):
    """d/dx of L = sum(O * G) by central differences of the forward oracle."""
    q, k, v, g = _inputs(1)
    scale = 0.7
    kw = _kw(var, q.shape[2], q.shape[1])
    dQ, dK, dV = oracle.attention_backward(q, k, v, g, scale, **kw)

    def loss(qq, kk, vv):
        O, _ = oracle.attention(qq, kk, vv, scale, **kw)
        return float((O * g).sum())

    eps = 1e-6
    for name, x, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[i] = (lp - lm) / (2 * eps)
        assert np.abs(num - grad).max() < 1e-6 * max(1.0, np.abs(grad).max()), name


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd(causal):
    """Dense and causal attention against PyTorch's CPU SDPA differentiated in
    float64 (a library routine, run, not copied); grouped heads are expanded
    for torch and their gradients summed back."""
    q, k, v, g = _inputs(2, B=2, H=4, Hkv=2, S=9, D=5)
    scale = 0.4
    dQ, dK, dV = oracle.attention_backward(q, k, v, g, scale, causal=causal)
    rep = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1),
        is_causal=causal, scale=scale)
    (out * torch.tensor(g)).sum().backward()
    for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


def test_gradient_identities():
    """Exact-derivative identities. Softmax rows sum to one, so the value
    gradients of a row add up to its output gradient: sum over keys of dV =
    sum over admitted rows of dout. A constant added to a row's scores leaves
    O unchanged, so the score gradients of a row sum to zero, and hence the
    key gradients sum to zero over keys (no mod, ALiBi). A row that admits a
    single key has O = that value, so its query gets no gradient."""
    q, k, v, g = _inputs(3, H=2, Hkv=2, S=7, D=4)
    for kw in (dict(), dict(causal=True), dict(causal=True, alibi_slopes=np.array([0.3, 0.1]))):
        dQ, dK, dV = oracle.attention_backward(q, k, v, g, 0.5, **kw)
        assert np.abs(dV.sum(axis=2) - g.sum(axis=2)).max() < 1e-12
        assert np.abs(dK.sum(axis=2)).max() < 1e-12
        if kw.get("causal"):
            assert np.abs(dQ[:, :, 0]).max() == 0.0          # row 0 admits key 0 only
    # linear in the output gradient
    a = oracle.attention_backward(q, k, v, g, 0.5, causal=True)
    b = oracle.attention_backward(q, k, v, 3.0 * g, 0.5, causal=True)
    for x, y in zip(a, b):
        assert np.abs(3.0 * x - y).max() < 1e-12


def test_fully_masked_rows_have_no_gradient():
    """With one key (label 0) and query rows 1-3 labelled 1, those rows admit
    nothing: O = 0 there, so they get no query gradient and add nothing to the
    key and value gradients; row 0 admits the single key with weight 1, so
    dV is its output gradient and dK is zero."""
    q, k, v, g = _inputs(4, H=1, Hkv=1, S=4, D=2)
    doc = np.array([[0, 1, 1, 1]])
    dQ, dK, dV = oracle.attention_backward(q, k[:, :, :1], v[:, :, :1], g, 1.0, causal=True,
                                           doc_ids=doc)
    assert np.abs(dQ).max() == 0.0
    assert np.abs(dK).max() == 0.0
    assert np.abs(dV - g[:, :, 0:1]).max() < 1e-15
