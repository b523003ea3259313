"""GPU parity of the attention backward (flexattn_bwd) against the fp64
oracle's gradients, on the same bf16 inputs and output gradient."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_tiled_attn_amd as fa
import oracle
from tests._parity import device_variant, oracle_kwargs, small, to_np
from workload import bf16_values, draw_dout

pytestmark = pytest.mark.gpu

# Tolerances, per tensor, relative to the reference's own size: the output is
# rounded to bf16 (at most 2^-8 relative), and P and dS enter the matrix
# products rounded to bf16 (at most 2^-8 relative each), so the largest error
# stays below about 3 * 2^-8 = 1.2e-2 of max|ref| and the mean error near
# 2^-8 of mean|ref|. Measured: at most 5.6e-3 and 2.5e-3.
REL_MAX = 1.5e-2
REL_MEAN = 5.0e-3


def say(msg):
    import sys
    print(msg, file=sys.stderr, flush=True)


def run_bwd(inp, block_mask="auto", seed=11):
    wl = inp.wl
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    dout = draw_dout(wl.B, wl.H, wl.Sq, wl.D, seed).to(torch.bfloat16).cuda()
    var = device_variant(inp)
    out, lse = fa.attention(q, k, v, var, scale=wl.scale)
    grads = fa.attention_backward(q, k, v, out, lse, dout, var, scale=wl.scale, block_mask=block_mask)
    torch.cuda.synchronize()
    return grads, dout


def ref_bwd(inp, dout):
    q, k, v = (bf16_values(t) for t in (inp.q, inp.k, inp.v))
    return oracle.attention_backward(q, k, v, bf16_values(dout.cpu()), inp.wl.scale,
                                     **oracle_kwargs(inp))


def check(inp, what, block_mask="auto"):
    say(f"[bwd] {what}")
    (dq, dk, dv), dout = run_bwd(inp, block_mask)
    ref = ref_bwd(inp, dout)
    stats = {}
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        g = to_np(got)
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        err = np.abs(g - want)
        scale_max = max(np.abs(want).max(initial=0.0), 1e-6)
        scale_mean = max(np.abs(want).mean() if want.size else 0.0, 1e-6)
        stats[name] = (err.max(initial=0.0) / scale_max, err.mean() / scale_mean)
        assert stats[name][0] <= REL_MAX and stats[name][1] <= REL_MEAN, f"{what}: {name} {stats}"
    say(f"[bwd]   " + " ".join(f"{n}: max {a:.2e} mean {b:.2e}" for n, (a, b) in stats.items()))
    return stats


VARIANTS = [
    dict(), dict(causal=True), dict(causal=True, window=48), dict(window=40),
    dict(documents=True), dict(documents=True, causal=True, window=64),
    dict(mod="alibi", causal=True), dict(mod="softcap", softcap=5.0),
    dict(mod="softcap", softcap=5.0, causal=True),
    dict(mod="relbias", rel_max=7), dict(mod="relbias", rel_max=1023, causal=True, window=90),
]


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: ",".join(f"{a}={b}" for a, b in v.items()) or "dense")
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_variants(var, D):
    check(small(S=200, D=D, **var), f"S=200 D={D} {var}")


@pytest.mark.parametrize("shape", [
    dict(S=1), dict(S=63), dict(S=64), dict(S=129), dict(S=333),
    dict(Sq=100, Skv=300), dict(Sq=300, Skv=100), dict(B=2, H=4, Hkv=2, S=260),
    dict(B=1, H=8, Hkv=1, S=150, causal=True),
], ids=lambda s: ",".join(f"{a}{b}" for a, b in s.items()))
def test_backward_shapes(shape):
    check(small(D=64, **shape), f"{shape}")


@pytest.mark.parametrize("case", [
    dict(Sq=1, Skv=300, q_offset=299, causal=True),
    dict(Sq=64, Skv=500, q_offset=436, causal=True, window=100, mod="alibi"),
    dict(Sq=200, Skv=700, q_offset=500, causal=True, documents=True),
    dict(Sq=150, Skv=150, q_offset=30, window=40, mod="softcap", softcap=5.0),
    dict(S=400, causal=True, prefix=150),
    dict(S=333, causal=True, prefix=129, window=90, documents=True),
    dict(Sq=100, Skv=600, q_offset=500, causal=True, prefix=256, mod="alibi"),
    dict(Sq=200, Skv=450, q_offset=250, causal=True, mod="relbias", rel_max=64),
], ids=lambda c: ",".join(f"{a}={b}" for a, b in c.items()))
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_offset_and_prefix(case, D):
    inp = small(D=D, H=4, Hkv=2, doc_range=(40, 300), **case)
    check(inp, f"D={D} {case}")
    (a, _), (b, _) = run_bwd(inp, "auto"), run_bwd(inp, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y), case


@pytest.mark.parametrize("D", [64, 128])
def test_backward_document_stage_list(D):
    """Documents with a causal mask over 4608 rows (18 query tiles): the
    dK/dV kernel reads the block-mask lists of up to 18 query tiles for a
    key tile (two passes of its parallel scan), skips the rows of other
    documents and treats tiles inside one document as full. The gradients
    equal, bit for bit, those computed without a block mask (every
    candidate row visited with the mask; that path meets the oracle in the
    tests above, and the oracle would take minutes at this size)."""
    inp = small(B=1, H=2, Hkv=1, S=4608, D=D, documents=True, causal=True, doc_range=(300, 2500))
    say(f"[bwd] S=4608 documents causal D={D}: block mask against none")
    (a, _), (b, _) = run_bwd(inp, "auto"), run_bwd(inp, None)
    for x, y in zip(a, b):
        assert torch.isfinite(x.float()).all()
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_documents_eight_slices(D):
    """Documents over eight (batch, head) slices, one per XCD's share of the
    grid, with GQA. The gradients meet the oracle and equal, bit for bit,
    those computed without a block mask."""
    inp = small(B=1, H=8, Hkv=2, S=1024, D=D, documents=True, causal=True, doc_range=(60, 400))
    check(inp, f"D={D} S=1024 H=8 documents")
    (a, _), (b, _) = run_bwd(inp, "auto"), run_bwd(inp, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_longer_causal_gqa():
    check(small(B=1, H=4, Hkv=2, S=1100, D=128, causal=True), "S=1100 causal GQA D=128")


def test_backward_head_dim_256_ragged():
    """D = 256 runs 32-row stages: a ragged tail, grouped heads and documents."""
    check(small(B=2, H=4, Hkv=2, S=333, D=256, causal=True, window=100), "S=333 D=256 causal window")
    check(small(B=1, H=2, S=290, D=256, documents=True, mod="alibi", doc_range=(30, 150)), "S=290 D=256 docs alibi")


@pytest.mark.parametrize("var", [dict(), dict(causal=True, window=150)],
                         ids=lambda v: ",".join(f"{a}={b}" for a, b in v.items()) or "plain")
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_recurring_document_labels(var, D):
    """Run j of the contiguous documents takes label j % 3: equal labels in
    several separate runs, so label equality alone decides the mask."""
    import dataclasses
    inp = small(S=500, D=D, documents=True, doc_range=(20, 140), **var)
    inp = dataclasses.replace(inp, doc_ids=(inp.doc_ids % 3).astype(np.int32))
    check(inp, f"recurring labels D={D} {var}")
    (a, _), (b, _) = run_bwd(inp, "auto"), run_bwd(inp, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y), var


@pytest.mark.parametrize("mod", ["none", "alibi"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_rows_with_no_admitted_key(mod, D):
    """300 query rows against 100 keys under documents: the rows whose
    document has no key are fully masked (LSE = -inf), so their P is 0 and
    their dQ rows are exactly zero."""
    inp = small(Sq=300, Skv=100, S=300, D=D, documents=True, doc_range=(20, 60), mod=mod)
    key_labels = set(inp.doc_ids[0, :100].tolist())
    empty = [i for i in range(300) if int(inp.doc_ids[0, i]) not in key_labels]
    assert len(empty) > 100
    check(inp, f"rows with no admitted key D={D} mod={mod}")
    (dq, dk, dv), _ = run_bwd(inp)
    assert torch.count_nonzero(dq[:, :, empty]).item() == 0


def test_backward_is_reproducible():
    """No atomics: two runs give identical bits."""
    inp = small(B=2, H=4, Hkv=2, S=300, D=128, causal=True)
    (a, _), (b, _) = run_bwd(inp), run_bwd(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_null_block_mask_is_bitwise_equal():
    # without any mask the kernels take the tiles inside Skv as full with no
    # block mask too (S = 300: two whole key tiles and a ragged one)
    for var in (dict(causal=True, window=70), dict(documents=True, causal=True), dict(),
                dict(mod="relbias", rel_max=7)):
        inp = small(S=300, D=64, **var)
        (a, _), (b, _) = run_bwd(inp, "auto"), run_bwd(inp, None)
        for x, y in zip(a, b):
            assert torch.equal(x, y), var


# ------------------------------------------------------------------ strided layouts
def _bshd(t):
    """The same values in a [B, S, H, D] buffer, viewed as [B, H, S, D]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _packed(*ts):
    """The tensors' values side by side in one [B, S, n, H, D + 8] buffer (a
    packed projection output with padded rows), each viewed as [B, H, S, D]."""
    B, H, S, D = ts[0].shape
    buf = torch.zeros((B, S, len(ts), H, D + 8), dtype=ts[0].dtype, device=ts[0].device)
    views = []
    for i, t in enumerate(ts):
        buf[:, :, i, :, :D] = t.transpose(1, 2)
        views.append(buf[:, :, i, :, :D].transpose(1, 2))
    return views


@pytest.mark.parametrize("var", [dict(causal=True), dict(documents=True, causal=True, window=64),
                                 dict(mod="relbias", rel_max=7)],
                         ids=lambda v: ",".join(f"{a}={b}" for a, b in v.items()))
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_strided_layouts(var, D):
    """Gradients of strided views ([B, S, H, D] buffers; q and the output
    gradient packed with padded rows) equal those of contiguous tensors bit
    for bit, and take the layout of their inputs."""
    say(f"[bwd] strided {var} D={D}")
    inp = small(B=2, H=4, Hkv=2, S=300, D=D, **var)
    wl = inp.wl
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    dout = draw_dout(wl.B, wl.H, wl.Sq, wl.D, 11).to(torch.bfloat16).cuda()
    dv_ = device_variant(inp)
    out, lse = fa.attention(q, k, v, dv_, scale=wl.scale)
    ref = fa.attention_backward(q, k, v, out, lse, dout, dv_, scale=wl.scale)
    qs, dos = _packed(q, dout)
    ks, vs = _bshd(k), _bshd(v)
    outs = torch.empty_strided(dos.shape, dos.stride(), dtype=out.dtype, device=out.device)
    outs.copy_(out)
    got = fa.attention_backward(qs, ks, vs, outs, lse, dos, dv_, scale=wl.scale)
    torch.cuda.synchronize()
    for name, a, b, like in zip(("dq", "dk", "dv"), ref, got, (qs, ks, vs)):
        assert b.stride() == like.stride(), name
        assert torch.equal(a, b), name


# ------------------------------------------------------------------ full size, as the bench runs it
@pytest.mark.parametrize("name,b,kvh", [("dense", 3, 5), ("causal_gqa", 1, 6)])
def test_backward_full_size_one_group(name, b, kvh):
    """The bench's backward (whole workload, one launch of each kernel, with
    the block mask of a masked variant and none for an unmasked one, as the
    bench runs them), checked on one batch row and one key/value head: the
    oracle's gradients of that slice (its query heads' dQ, the head's dK and
    dV) are exact, since no other slice feeds them."""
    from workload import WORKLOADS, make_inputs
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    say(f"[bwd] full-size {name}: gpu")
    bm = "auto" if device_variant(inp).mask_kind else None
    (dq, dk, dv), dout = run_bwd(inp, block_mask=bm, seed=wl.seed)
    rep = wl.H // wl.Hkv
    heads = list(range(kvh * rep, (kvh + 1) * rep))
    q = bf16_values(inp.q[b:b + 1, heads])
    k = bf16_values(inp.k[b:b + 1, kvh:kvh + 1])
    v = bf16_values(inp.v[b:b + 1, kvh:kvh + 1])
    g = bf16_values(dout[b:b + 1, heads].cpu())
    say(f"[bwd] full-size {name}: oracle on batch {b}, kv head {kvh} ({rep} query heads)")
    ref = oracle.attention_backward(q, k, v, g, wl.scale, causal=wl.causal)
    got = (to_np(dq[b:b + 1, heads]), to_np(dk[b:b + 1, kvh:kvh + 1]), to_np(dv[b:b + 1, kvh:kvh + 1]))
    for nm, gt, want in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(gt - want)
        rmax = err.max() / max(np.abs(want).max(), 1e-6)
        rmean = err.mean() / max(np.abs(want).mean(), 1e-6)
        say(f"[bwd]   {nm}: max {rmax:.2e} mean {rmean:.2e}")
        assert rmax <= REL_MAX and rmean <= REL_MEAN, (name, nm, rmax, rmean)
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any().item()


# ------------------------------------------------------------------ broadcast (overlapping) inputs
def test_backward_expanded_kv():
    """K and V expanded over the batch (stride 0): the C ABI refuses the
    layout for the gradients (they would collide), and the binding copies
    such inputs first, giving the per-batch gradients of the view, bit for
    bit those of the contiguous call."""
    inp = small(B=3, H=4, Hkv=2, S=150, D=64, causal=True)
    wl = inp.wl
    q = inp.q.cuda()
    k1, v1 = inp.k[:1].cuda(), inp.v[:1].cuda()
    kb, vb = k1.expand(3, -1, -1, -1), v1.expand(3, -1, -1, -1)
    assert kb.stride(0) == 0 and not fa.non_overlapping(kb)
    var = fa.Variant(causal=True)
    out, lse = fa.attention(q, kb, vb, var, scale=wl.scale)
    dout = draw_dout(wl.B, wl.H, wl.Sq, wl.D, 5).to(torch.bfloat16).cuda()
    # the raw entry point with the expanded strides: rejected before any launch
    p = fa.make_params(var, torch.bfloat16)
    fa.set_layout(p, q, kb, vb, out)
    dk = torch.empty(1, 2, 150, 64, dtype=torch.bfloat16, device="cuda").expand(3, -1, -1, -1)
    dq, dv = torch.empty_like(q), torch.empty_like(dk)
    delta = torch.empty(3, 4, 150, dtype=torch.float32, device="cuda")
    st = fa.flexattn_bwd(q, kb, vb, out, lse, dout, dq, dk, dv, delta, 3, 4, 2, 150, 150, 64, wl.scale,
                         var.mask_kind, var.mod_kind, p, None, check=False)
    assert st == fa._lib.ERR_ARG
    # the binding: gradients of the view, equal to the contiguous call's
    got = fa.attention_backward(q, kb, vb, out, lse, dout, var, scale=wl.scale)
    ref = fa.attention_backward(q, kb.contiguous(), vb.contiguous(), out, lse, dout, var, scale=wl.scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert fa.non_overlapping(a), name
        assert torch.equal(a, b), name
