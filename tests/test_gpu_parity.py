"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Small shapes and every full-size workload are compared element by element over
the whole output (the full sizes against the oracle run in a pool of host
processes). Tolerances: O max-abs 2e-2 and mean-abs 2e-3, LSE 1e-3; rows with no
admitted key must be O = 0 and LSE = -inf on both sides.
"""
import sys

import numpy as np
import pytest
import torch

import attention_tiled_attn_amd as fa
import oracle
from tests._parity import (check_pair_lists, compare, device_variant, make_inputs, run_gpu, run_oracle,
                           run_oracle_full, small, to_np)
from workload import WORKLOADS

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_full(inp, block_mask="auto", what=""):
    say(f"[parity] {what} B={inp.wl.B} H={inp.wl.H} Hkv={inp.wl.Hkv} Sq={inp.wl.Sq} "
        f"Skv={inp.wl.Skv} D={inp.wl.D} {inp.wl.dtype} causal={inp.wl.causal} "
        f"window={inp.wl.window} docs={inp.doc_ids is not None} mod={inp.wl.mod}")
    O, L = run_gpu(inp, block_mask)
    Oref, Lref = run_oracle(inp)
    return compare(to_np(O), to_np(L), Oref, Lref, what)


# ------------------------------------------------------------------ the tiny workload, whole
def test_tiny_causal_fp32():
    inp = make_inputs(WORKLOADS["tiny_causal"])
    check_full(inp, what="tiny_causal")
    # Reported, not gated: the kernel rounds the fp32 inputs to bf16 on load
    # (both products run on bf16 matrix cores), so the distance to the oracle
    # on the unrounded fp32 values holds that input rounding too.
    O, L = run_gpu(inp)
    q, k, v = (t.double().numpy() for t in (inp.q, inp.k, inp.v))
    Oref, Lref = oracle.attention(q, k, v, inp.wl.scale, causal=True)
    e = np.abs(to_np(O) - Oref)
    print(f"[parity] tiny_causal fp32 vs oracle on unrounded fp32 inputs: O max-abs {e.max():.3e} "
          f"mean-abs {e.mean():.3e}, LSE max-abs {np.abs(to_np(L) - Lref).max():.3e} (not gated)")


# ------------------------------------------------------------------ shapes x variants
SHAPES = [
    dict(S=1), dict(S=2), dict(S=3), dict(S=127), dict(S=129), dict(S=200), dict(S=333),
    dict(S=256, D=128), dict(S=200, D=128), dict(S=300, H=4, Hkv=2), dict(S=260, H=4, Hkv=1, D=128),
    dict(Sq=100, Skv=300, S=300), dict(Sq=300, Skv=100, S=300), dict(S=190, B=2, H=2),
]
VARIANTS = [
    dict(), dict(causal=True), dict(causal=True, window=50), dict(window=70),
    dict(documents=True), dict(documents=True, causal=True, window=40),
    dict(causal=True, mod="alibi"), dict(mod="alibi"), dict(mod="softcap", softcap=5.0),
    dict(causal=True, mod="softcap", softcap=30.0), dict(documents=True, mod="alibi", causal=True),
    dict(mod="relbias", rel_max=5), dict(causal=True, mod="relbias", rel_max=1023),
    dict(documents=True, causal=True, window=40, mod="relbias", rel_max=17),
]


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: ",".join(f"{k}={x}" for k, x in v.items()) or "dense")
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: ",".join(f"{k}{x}" for k, x in s.items()))
def test_small_shapes(shape, var):
    inp = small(**shape, **var)
    check_full(inp, what=f"{shape} {var}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_dtypes_and_head_dims(dtype, D):
    check_full(small(S=257, D=D, dtype=dtype, causal=True, seed=11), what=f"{dtype} D{D}")


# ------------------------------------------------------------------ GPU-side invariants
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("R", [0, 3, 1023])
def test_relative_bias_fp32_path(D, R):
    """fp32 inputs run the 128-row kernel; its bias table is staged the same way."""
    inp = small(S=300, D=D, dtype="fp32", causal=True, mod="relbias", rel_max=R)
    check_full(inp, what=f"fp32 relbias D={D} R={R}")


def test_null_block_mask_is_bitwise_equal():
    # the last two have padding rows past Sq in waves with real rows, beside
    # full tiles: the padding rows must not sway the rescale of the real ones
    for var in (dict(causal=True), dict(documents=True, causal=True, window=60), dict(), dict(mod="alibi"),
                dict(S=1800, documents=True, causal=True, window=300, doc_range=(60, 700)),
                dict(S=1000, documents=True, mod="softcap", softcap=5.0, doc_range=(60, 700))):
        var = {"S": 520, **var}
        inp = small(D=128, **var)
        O1, L1 = run_gpu(inp, block_mask="auto")
        O2, L2 = run_gpu(inp, block_mask=None)
        assert torch.equal(O1, O2) and torch.equal(L1, L2), var


LONGEST_FIRST_CASES = [
    # document masks with B*H a multiple of 8 take their query tiles longest
    # first within each XCD; uneven documents give the tiles uneven work
    dict(B=1, H=8, S=1800, D=128, causal=True, window=300),
    dict(B=2, H=4, Hkv=2, S=1100, D=64),
    dict(B=4, H=4, S=600, D=128, causal=True),
    dict(B=1, H=8, S=900, D=256, causal=True, mod="alibi"),
]


@pytest.mark.parametrize("case", LONGEST_FIRST_CASES,
                         ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_document_items_longest_first(case):
    """Every query tile is computed exactly once under the reordered mapping
    (outputs start as NaN), matches the oracle, and is bitwise equal to the
    unordered mapping that runs without a block mask."""
    inp = small(documents=True, doc_range=(60, 700), **case)
    check_full(inp, what=f"longest-first {case}")
    O1, L1 = run_gpu(inp, block_mask="auto")
    O2, L2 = run_gpu(inp, block_mask=None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def recurring_labels(inp, period=3):
    """The same inputs with document labels that come back: run j of the
    contiguous documents takes label j % period, so equal labels lie in
    several separate runs (label equality alone decides the mask)."""
    import dataclasses
    return dataclasses.replace(inp, doc_ids=(inp.doc_ids % period).astype(np.int32))


@pytest.mark.parametrize("var", [dict(), dict(causal=True), dict(causal=True, window=150),
                                 dict(causal=True, mod="alibi")],
                         ids=lambda v: ",".join(f"{k}={x}" for k, x in v.items()) or "plain")
@pytest.mark.parametrize("D", [64, 128, 256])
def test_recurring_document_labels(var, D):
    inp = recurring_labels(small(S=700, D=D, documents=True, doc_range=(20, 140), **var))
    labels = inp.doc_ids[0]
    starts = np.flatnonzero(np.diff(labels) != 0) + 1
    assert len(set(labels.tolist())) < len(starts) + 1   # some label spans several runs
    check_full(inp, "auto", f"recurring labels D={D} {var}")
    O1, L1 = run_gpu(inp, "auto")
    O2, L2 = run_gpu(inp, None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_repeat_runs_are_bitwise_equal():
    inp = small(S=700, D=128, causal=True, mod="alibi", H=4, Hkv=2)
    O1, L1 = run_gpu(inp)
    O2, L2 = run_gpu(inp)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_gqa_equals_repeated_heads_bitwise():
    inp = small(S=384, D=128, H=8, Hkv=2, causal=True)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    O1, L1 = run_gpu(inp, qkv=(q, k, v))
    rep = 4
    k2 = k.repeat_interleave(rep, dim=1).contiguous()
    v2 = v.repeat_interleave(rep, dim=1).contiguous()
    var = device_variant(inp)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.attention(q, k2, v2, var, scale=inp.wl.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(O1, out) and torch.equal(L1, lse)


def test_fully_masked_rows():
    """Queries past Skv whose document has no key at all: O = 0, LSE = -inf."""
    inp = small(Sq=400, Skv=150, S=400, documents=True, causal=True, doc_range=(40, 90))
    O, L = run_gpu(inp)
    Oref, Lref = run_oracle(inp)
    assert np.isneginf(Lref).any()
    compare(to_np(O), to_np(L), Oref, Lref, "fully masked rows")


def test_lse_optional():
    inp = small(S=300, causal=True)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    out, lse = fa.attention(q, k, v, fa.Variant(causal=True), scale=inp.wl.scale, with_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    Oref, _ = run_oracle(inp)
    err = np.abs(to_np(out) - Oref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_split_kv_merge_identity():
    """Attention over two key halves, merged by their LSEs, equals attention
    over all keys (the identity a sharded-over-keys run would use)."""
    inp = small(S=512, D=128, H=2, seed=21)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    var = fa.Variant()
    O, L = fa.attention(q, k, v, var, scale=inp.wl.scale)
    n = 200
    O1, L1 = fa.attention(q, k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), var, scale=inp.wl.scale)
    O2, L2 = fa.attention(q, k[:, :, n:].contiguous(), v[:, :, n:].contiguous(), var, scale=inp.wl.scale)
    Lm = torch.logaddexp(L1, L2)
    Om = torch.exp(L1 - Lm)[..., None] * O1.float() + torch.exp(L2 - Lm)[..., None] * O2.float()
    torch.cuda.synchronize()
    assert (Lm - L).abs().max().item() < 1e-4
    assert (Om - O.float()).abs().max().item() < 2e-2


# ------------------------------------------------------------------ query offset and prefix-LM
# Decoding and chunked prefill: Sq queries after Skv - Sq cached keys, so
# q_offset = Skv - Sq; prefix-LM: keys below the prefix seen by every query.
OFFSET_CASES = [
    dict(Sq=1, Skv=300, q_offset=299, causal=True),
    dict(Sq=5, Skv=1000, q_offset=995, causal=True, mod="alibi"),
    dict(Sq=64, Skv=777, q_offset=713, causal=True, window=100),
    dict(Sq=300, Skv=1000, q_offset=700, causal=True, documents=True),
    dict(Sq=257, Skv=513, q_offset=256, causal=True, mod="softcap", softcap=5.0),
    dict(Sq=200, Skv=640, q_offset=77, causal=True, window=150, documents=True, mod="alibi"),
    dict(Sq=130, Skv=130, q_offset=40, window=30),                 # window only, offset
    dict(S=600, causal=True, prefix=200),
    dict(S=333, causal=True, prefix=129, window=100),
    dict(S=500, causal=True, prefix=300, documents=True),
    dict(S=300, causal=True, prefix=1000, mod="alibi"),            # prefix past the end: dense
    dict(Sq=100, Skv=700, q_offset=600, causal=True, prefix=256, mod="softcap", softcap=5.0),
    dict(Sq=64, Skv=500, q_offset=436, causal=True, mod="relbias", rel_max=100),
]


@pytest.mark.parametrize("case", OFFSET_CASES, ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
@pytest.mark.parametrize("D", [64, 128])
def test_offset_and_prefix(case, D):
    inp = small(D=D, doc_range=(40, 300), **case)
    check_full(inp, what=f"D={D} {case}")
    # the block mask must not change a single bit
    O1, L1 = run_gpu(inp)
    O2, L2 = run_gpu(inp, block_mask=None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("case", OFFSET_CASES, ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_block_mask_offset_and_prefix(case):
    inp = small(doc_range=(40, 300), **case)
    wl = inp.wl
    bm = fa.build_block_mask(device_variant(inp), wl.B, wl.Sq, wl.Skv)
    torch.cuda.synchronize()
    counts, lists = bm.counts().cpu().numpy(), bm.lists().cpu().numpy()
    for b in range(counts.shape[0]):
        doc_row = None if inp.doc_ids is None else inp.doc_ids[b]
        ref = oracle.tile_classes(wl.Sq, wl.Skv, 128, causal=wl.causal, window=wl.window or None,
                                  doc_row=doc_row, q_offset=wl.q_offset, prefix=wl.prefix)
        check_pair_lists(counts[b], lists[b], ref)


# ------------------------------------------------------------------ block-mask builder
@pytest.mark.parametrize("case", [
    dict(S=1000, causal=True), dict(S=1000, causal=True, window=300), dict(S=777, window=200),
    dict(S=1300, documents=True), dict(S=1300, documents=True, causal=True, window=256),
    dict(Sq=500, Skv=900, S=900, causal=True), dict(S=640),
])
def test_block_mask_matches_tile_classes(case):
    inp = small(**case, doc_range=(50, 400))
    wl = inp.wl
    var = device_variant(inp)
    bm = fa.build_block_mask(var, wl.B, wl.Sq, wl.Skv)
    torch.cuda.synchronize()
    counts, lists = bm.counts().cpu().numpy(), bm.lists().cpu().numpy()
    for b in range(counts.shape[0]):
        doc_row = None if inp.doc_ids is None else inp.doc_ids[b]
        ref = oracle.tile_classes(wl.Sq, wl.Skv, 128, causal=wl.causal, window=wl.window or None,
                                  doc_row=doc_row)
        check_pair_lists(counts[b], lists[b], ref)


def test_block_mask_document_workload_full_size():
    inp = make_inputs(WORKLOADS["doc_swa"])
    wl = inp.wl
    bm = fa.build_block_mask(device_variant(inp), wl.B, wl.Sq, wl.Skv)
    torch.cuda.synchronize()
    counts, lists = bm.counts().cpu().numpy(), bm.lists().cpu().numpy()
    ref = oracle.tile_classes(wl.Sq, wl.Skv, 128, causal=True, window=wl.window, doc_row=inp.doc_ids[0])
    check_pair_lists(counts[0], lists[0], ref)
    say(f"[blockmask] doc_swa: {int((ref == 2).sum())} full + {int((ref == 1).sum())} partial "
        f"half-tiles of {ref.size}, lists equal to the oracle's classes")


@pytest.mark.parametrize("case", [
    dict(S=1300), dict(S=1300, causal=True), dict(S=1300, causal=True, window=256),
    dict(S=900, window=200), dict(Sq=500, Skv=1100, q_offset=600, causal=True),
    dict(S=1000, causal=True, prefix=300), dict(S=1000, causal=True, prefix=300, window=200),
    dict(Sq=333, Skv=777, q_offset=100, window=150, B=2),
], ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
@pytest.mark.parametrize("period,runs", [(3, (50, 400)), (2, (5, 40)), (4, (1, 3))],
                         ids=["long runs", "short runs", "runs of 1-3"])
def test_block_mask_recurring_labels_exact(case, period, runs):
    """Labels that come back in separate runs (run j takes label j % period):
    the label ranges of a half and a key tile overlap without deciding
    whether a pair is admitted, and the builder's exact test must give the
    oracle's classes."""
    inp = recurring_labels(small(documents=True, doc_range=runs, **case), period)
    wl = inp.wl
    bm = fa.build_block_mask(device_variant(inp), wl.B, wl.Sq, wl.Skv)
    torch.cuda.synchronize()
    counts, lists = bm.counts().cpu().numpy(), bm.lists().cpu().numpy()
    for b in range(counts.shape[0]):
        ref = oracle.tile_classes(wl.Sq, wl.Skv, 128, causal=wl.causal, window=wl.window or None,
                                  doc_row=inp.doc_ids[b], q_offset=wl.q_offset, prefix=wl.prefix)
        check_pair_lists(counts[b], lists[b], ref)


# ------------------------------------------------------------------ full-size workloads
# Every element of O and LSE, against the oracle run over the whole tensors in
# a pool of host processes, in the launch configuration the benchmark times
# (the library's own block mask for a masked variant, none for an unmasked
# one, whose key tiles are then taken as full). The long-context workloads hold 34e9 scores
# each; the oracle takes about half a minute for one on the GPU host.
WHOLE = ["dense", "causal_gqa", "doc_swa", "causal_gqa_shard8", "prefix_lm", "chunked_prefill",
         "relbias", "causal_gqa_d256", "alibi_d64", "alibi_d128", "softcap_d64", "softcap_d128"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", WHOLE)
def test_full_size_whole(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    say(f"[parity] full-size {name}, whole tensors: gpu")
    O, L = run_gpu(inp, block_mask="auto" if device_variant(inp).mask_kind else None)
    # every element written (outputs were NaN-filled)
    assert not torch.isnan(O).any().item() and not torch.isnan(L).any().item()
    Og, Lg = to_np(O), to_np(L)
    del O, L
    st = {}
    Oref, Lref = run_oracle_full(inp, stats=st)
    stats = compare(Og, Lg, Oref, Lref, name)
    say(f"[parity] {name}: {stats}; oracle {st['seconds']:.1f} s on {st['workers']} processes")


# ------------------------------------------------------------------ strided layouts
def _bshd(t: torch.Tensor) -> torch.Tensor:
    """The same values in a [B, S, H, D] buffer, viewed as [B, H, S, D]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("case", [
    dict(S=300, D=64), dict(S=257, D=128, causal=True),
    dict(B=2, H=4, Hkv=2, S=333, D=128, causal=True, window=100),
    dict(B=2, H=4, Hkv=1, S=200, D=64, documents=True, mod="alibi"),
    dict(Sq=70, Skv=400, q_offset=330, D=128, causal=True, mod="relbias", rel_max=50),
    dict(S=190, D=64, dtype="fp32", causal=True), dict(S=260, D=128, dtype="fp32"),
], ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_strided_layouts_match_contiguous_bitwise(case):
    """[B, S, H, D] buffers viewed as [B, H, S, D] (q, k, v and out) give the
    contiguous call's bits, and the oracle's values."""
    inp = small(doc_range=(30, 150), **case)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    O1, L1 = run_gpu(inp, qkv=(q, k, v))
    qs, ks, vs = _bshd(q), _bshd(k), _bshd(v)
    assert not qs.is_contiguous() and qs.stride(3) == 1
    out = _bshd(torch.full_like(q, float("nan")))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.attention(qs, ks, vs, device_variant(inp), scale=inp.wl.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, O1) and torch.equal(lse, L1)
    Oref, Lref = run_oracle(inp)
    compare(to_np(out), to_np(lse), Oref, Lref, f"strided {case}")


def test_strided_kv_shared_across_batch():
    """Batch stride 0 for K and V: every batch row reads the same keys."""
    inp = small(B=3, H=2, S=150, D=64, causal=True)
    q = inp.q.cuda()
    k1, v1 = inp.k[:1].cuda(), inp.v[:1].cuda()
    kb, vb = k1.expand(3, -1, -1, -1), v1.expand(3, -1, -1, -1)
    assert kb.stride(0) == 0
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.attention(q, kb, vb, fa.Variant(causal=True), scale=inp.wl.scale, out=out, lse=lse)
    ref_out, ref_lse = fa.attention(q, kb.contiguous(), vb.contiguous(), fa.Variant(causal=True),
                                    scale=inp.wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


# ------------------------------------------------------------------ head dimension 256
D256_CASES = [
    dict(S=1), dict(S=33), dict(S=200), dict(S=333, causal=True),
    dict(S=513, H=4, Hkv=2, causal=True, window=100), dict(S=300, documents=True, causal=True),
    dict(S=260, mod="alibi", causal=True), dict(S=260, mod="softcap", softcap=5.0),
    dict(S=260, mod="relbias", rel_max=50, causal=True), dict(S=290, documents=True, mod="alibi"),
    dict(Sq=70, Skv=400, q_offset=330, causal=True), dict(S=300, causal=True, prefix=100),
]


@pytest.mark.parametrize("case", D256_CASES, ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_head_dim_256(case):
    inp = small(D=256, doc_range=(30, 150), **case)
    check_full(inp, what=f"D=256 {case}")
    O1, L1 = run_gpu(inp)
    O2, L2 = run_gpu(inp, block_mask=None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_head_dim_256_strided_and_decode():
    inp = small(B=2, H=8, Hkv=2, Sq=3, Skv=700, q_offset=697, D=256, causal=True)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    O1, L1 = run_gpu(inp, qkv=(q, k, v))
    qs, ks, vs = (_bshd(t) for t in (q, k, v))
    O2, L2 = fa.attention(qs, ks, vs, device_variant(inp), scale=inp.wl.scale)
    O3, L3 = fa.decode(q, k, v, device_variant(inp), scale=inp.wl.scale, splits=3)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    Oref, Lref = run_oracle(inp)
    compare(to_np(O3), to_np(L3), Oref, Lref, "D=256 decode")


# ------------------------------------------------------------------ maximum key-list lengths
@pytest.mark.parametrize("Skv", [2048 * 128, 2048 * 128 + 77], ids=["2048 tiles", "past 2048 tiles"])
@pytest.mark.parametrize("causal", [False, True])
def test_maximum_key_lists(Skv, causal):
    """The ping-pong kernel's longest key-tile list (2048 tiles of 128 keys)
    and one key past it, where bf16 inputs go to the 128-row kernel; every
    query row is compared with the oracle."""
    Sq = 64
    inp = small(B=1, H=2, Hkv=1, Sq=Sq, Skv=Skv, D=64, causal=causal,
                q_offset=(Skv - Sq) if causal else 0)
    check_full(inp, what=f"Skv={Skv} causal={causal}")


def test_decode_maximum_key_list():
    """Decoding at the longest cache the forward takes (2048 key tiles), the
    library's split count, against the oracle."""
    Skv = 2048 * 128
    inp = small(B=1, H=4, Hkv=1, Sq=1, Skv=Skv, D=128, causal=True, q_offset=Skv - 1)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    O, L = fa.decode(q, k, v, device_variant(inp), scale=inp.wl.scale)
    torch.cuda.synchronize()
    Oref, Lref = run_oracle(inp)
    compare(to_np(O), to_np(L), Oref, Lref, "decode, 2048 key tiles")
