"""GPU parity of the decode entry point (flexattn_decode): query heads packed
per key/value head and the key range split over workgroups, against the fp64
oracle, for the variants and layouts flexattn_fwd takes."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import attention_tiled_attn_amd as fa
from tests._parity import compare, device_variant, run_oracle, small, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_decode(inp, splits, block_mask="auto", layout="contiguous"):
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    if layout == "bshd":
        q, k, v = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.decode(q, k, v, device_variant(inp), scale=inp.wl.scale, splits=splits, out=out, lse=lse,
              block_mask=block_mask)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    dict(B=2, H=8, Hkv=2, Sq=1, Skv=1000, q_offset=999, causal=True),
    dict(B=1, H=32, Hkv=8, Sq=1, Skv=4099, q_offset=4098, causal=True, D=128),
    dict(B=3, H=4, Hkv=1, Sq=5, Skv=777, q_offset=772, causal=True, mod="alibi"),
    dict(B=1, H=8, Hkv=8, Sq=1, Skv=600, q_offset=599, causal=True, mod="softcap", softcap=5.0),
    dict(B=2, H=16, Hkv=2, Sq=16, Skv=2000, q_offset=1984, causal=True, window=700, D=128),
    dict(B=1, H=8, Hkv=2, Sq=3, Skv=1500, q_offset=1497, causal=True, documents=True),
    dict(B=1, H=4, Hkv=2, Sq=2, Skv=900, q_offset=898, causal=True, prefix=300, mod="relbias", rel_max=40),
    dict(B=2, H=2, Hkv=1, Sq=1, Skv=50, q_offset=49, causal=True),        # one short key tile
    dict(B=1, H=4, Hkv=4, Sq=64, Skv=640, D=128),                          # no mask, 64 rows each
    dict(B=1, H=8, Hkv=1, Sq=32, Skv=300, q_offset=268, causal=True, D=64),  # 256 packed rows
]


@pytest.mark.parametrize("splits", [1, 3, None])
@pytest.mark.parametrize("case", CASES, ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_decode_matches_oracle(case, splits):
    inp = small(doc_range=(100, 600), **case)
    say(f"[decode] {case} splits={splits}")
    O, L = run_decode(inp, splits)
    Oref, Lref = run_oracle(inp)
    compare(to_np(O), to_np(L), Oref, Lref, f"decode {case} splits={splits}")


def test_decode_more_splits_than_tiles():
    """Splits that get no key tile write empty partial results (O = 0,
    LSE = -inf) that the merge ignores."""
    inp = small(B=1, H=4, Hkv=2, Sq=2, Skv=200, q_offset=198, causal=True, window=3)
    O, L = run_decode(inp, 7)
    Oref, Lref = run_oracle(inp)
    compare(to_np(O), to_np(L), Oref, Lref, "decode many splits")


@pytest.mark.parametrize("layout", ["bshd"])
def test_decode_strided_and_null_block_mask(layout):
    inp = small(B=2, H=8, Hkv=2, Sq=4, Skv=1100, q_offset=1096, D=128, causal=True, mod="alibi")
    O1, L1 = run_decode(inp, 3)
    O2, L2 = run_decode(inp, 3, layout=layout)
    O3, L3 = run_decode(inp, 3, block_mask=None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.equal(O1, O3) and torch.equal(L1, L3)


def test_decode_agrees_with_forward():
    """The decode path and flexattn_fwd compute the same attention (different
    summation order: close, not bitwise)."""
    inp = small(B=2, H=16, Hkv=4, Sq=1, Skv=3000, q_offset=2999, D=128, causal=True)
    O, L = run_decode(inp, None)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    Of, Lf = fa.attention(q, k, v, device_variant(inp), scale=inp.wl.scale)
    torch.cuda.synchronize()
    assert (O.float() - Of.float()).abs().max().item() < 1e-2
    assert (L - Lf).abs().max().item() < 1e-4


def test_decode_workload_full_size_sampled():
    """The bench's decode step (16 sequences x 32 heads, 32767 cached keys,
    the library's split count), checked against the oracle on sampled
    (batch, head) pairs; every output element written."""
    from workload import WORKLOADS, make_inputs
    import oracle
    from workload import bf16_values
    wl = WORKLOADS["decode"]
    inp = make_inputs(wl)
    O, L = run_decode(inp, None)
    for b, heads in ((0, [0, 5, 31]), (9, [12, 13]), (15, [31])):
        q, k, v = (bf16_values(t[b:b + 1]) for t in (inp.q, inp.k, inp.v))
        Oref, Lref = oracle.attention(q, k, v, wl.scale, causal=True, q_offset=wl.q_offset, heads=heads)
        compare(to_np(O[b:b + 1, heads]), to_np(L[b:b + 1, heads]), Oref[:, heads], Lref[:, heads],
                f"decode full size b={b}")
    assert not torch.isnan(O).any().item() and not torch.isnan(L).any().item()


# ------------------------------------------------------------------ split key lists (rep * Sq > 256)
TILE_SPLIT_CASES = [
    dict(B=1, H=2, Hkv=1, Sq=300, Skv=300, causal=True),
    dict(B=2, H=4, Hkv=2, S=700, D=128, causal=True, window=200),
    dict(B=1, H=2, S=900, documents=True, causal=True, mod="alibi"),
    dict(B=1, H=4, Hkv=4, Sq=500, Skv=1300, q_offset=800, causal=True, mod="softcap", softcap=5.0),
    dict(B=1, H=2, S=600, causal=True, prefix=200, mod="relbias", rel_max=50),
    dict(B=1, H=2, S=520, D=256, causal=True),
    dict(B=1, H=2, S=400, D=128),
    # Sq <= 128 with rep * Sq > 256: the split lists of the key-split mapping
    dict(B=1, H=8, Hkv=2, Sq=100, Skv=1500, q_offset=1400, causal=True, D=128),
    dict(B=2, H=4, Hkv=1, Sq=128, Skv=900, q_offset=772, causal=True, documents=True, mod="alibi"),
]


@pytest.mark.parametrize("splits", [2, 5, None])
@pytest.mark.parametrize("case", TILE_SPLIT_CASES, ids=lambda c: ",".join(f"{k}={x}" for k, x in c.items()))
def test_split_tiles_match_oracle(case, splits):
    """More rows than one workgroup packs: every 256-row query tile's key list
    is cut into `splits` parts, merged as in decoding (outputs start as NaN,
    so every element is written)."""
    inp = small(doc_range=(60, 400), **case)
    say(f"[split] {case} splits={splits}")
    O, L = run_decode(inp, splits)
    Oref, Lref = run_oracle(inp)
    compare(to_np(O), to_np(L), Oref, Lref, f"split tiles {case} splits={splits}")


def test_split_tiles_strided_null_mask_and_forward():
    """Unpacked splits: [B, S, H, D] views give the same bits. Without a
    block mask the splits cut the list of every key tile rather than of the
    admitted ones, so the parts (and the merge's rounding) differ: that run,
    like flexattn_fwd (one part), agrees closely, not bitwise."""
    inp = small(B=2, H=4, Hkv=2, S=900, D=128, causal=True, mod="alibi")
    O1, L1 = run_decode(inp, 3)
    O2, L2 = run_decode(inp, 3, layout="bshd")
    O3, L3 = run_decode(inp, 3, block_mask=None)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    Of, Lf = fa.attention(q, k, v, device_variant(inp), scale=inp.wl.scale)
    torch.cuda.synchronize()
    for Ox, Lx in ((O3, L3), (Of, Lf)):
        assert (O1.float() - Ox.float()).abs().max().item() < 1e-2
        assert (L1 - Lx).abs().max().item() < 1e-4
    Oref, Lref = run_oracle(inp)
    compare(to_np(O3), to_np(L3), Oref, Lref, "split tiles, no block mask")


def test_split_tiles_full_size_sampled():
    """causal_gqa_shard8 (2 x 4 query heads, 1 key/value head, 8192 rows:
    256 query tiles for 256 CUs) through the split path with the library's
    split count, checked against the oracle on sampled rows of every head."""
    from workload import WORKLOADS, bf16_values, make_inputs
    import oracle
    wl = WORKLOADS["causal_gqa_shard8"]
    assert fa.flexattn_split_count(wl.B, wl.H, wl.Hkv, wl.Sq, wl.Skv) > 1
    inp = make_inputs(wl)
    O, L = run_decode(inp, None)
    rows = np.r_[0:40, 4000:4040, 8150:8192]
    for b in range(wl.B):
        q, k, v = (bf16_values(t[b:b + 1]) for t in (inp.q, inp.k, inp.v))
        Oref, Lref = oracle.attention(q, k, v, wl.scale, causal=True, rows=rows)
        compare(to_np(O[b:b + 1, :, rows]), to_np(L[b:b + 1, :, rows]), Oref, Lref, f"shard8 split b={b}")
    assert not torch.isnan(O).any().item() and not torch.isnan(L).any().item()
