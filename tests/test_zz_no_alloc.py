"""flexattn_decode_static, the decode entry point that allocates nothing (its
split results go to the library's static scratch), against flexattn_decode
with a caller workspace: the same kernels, so the same bits, and both within
the oracle's tolerances. Two calls in a row share the scratch; the second is
smaller than the first, and must not see anything the first left behind."""
import numpy as np
import pytest
import torch

import attention_tiled_attn_amd as fa
from tests._parity import compare, device_variant, run_oracle, small, to_np

pytestmark = pytest.mark.gpu


def _both(inp, splits):
    """(O, LSE) from flexattn_decode_static and from flexattn_decode, called
    through the C ABI with the same arguments (outputs NaN-filled first)."""
    wl = inp.wl
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    B, H, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    var = device_variant(inp)
    bm = fa.build_block_mask(var, B, Sq, Skv, q.device)
    p = fa.make_params(var, q.dtype)
    fa.set_layout(p, q, k, v, q)
    res = []
    for static in (True, False):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=q.device)
        if static:
            fa.flexattn_decode_static(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, wl.scale, var.mask_kind,
                                      var.mod_kind, p, bm.struct, splits)
        else:
            nbytes = fa.flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits)
            ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=q.device)
            fa.flexattn_decode(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, wl.scale, var.mask_kind,
                               var.mod_kind, p, bm.struct, splits, ws, nbytes)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


# first call larger than the second; packed decoding (rep * Sq <= 256) and
# split query-tile lists (rep * Sq > 256)
SEQUENCES = [
    [(dict(B=4, H=16, Hkv=4, Sq=1, Skv=5000, D=128, causal=True, q_offset=4999), 4),
     (dict(B=2, H=8, Hkv=2, Sq=3, Skv=1200, D=64, causal=True, q_offset=1197, mod="alibi"), 3)],
    [(dict(B=1, H=4, Hkv=1, Sq=700, Skv=2100, D=128, causal=True, q_offset=1400), 3),
     (dict(B=1, H=2, Hkv=1, Sq=300, Skv=900, D=128, documents=True, doc_range=(50, 300)), 2)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["packed", "split-lists"])
def test_decode_static_matches_workspace_entry(seq):
    for case, splits in seq:
        inp = small(**case)
        print(f"[no-alloc] {case} splits={splits}", flush=True)
        (Os, Ls), (Ow, Lw) = _both(inp, splits)
        assert not torch.isnan(Os).any().item() and not torch.isnan(Ls).any().item()
        assert torch.equal(Os, Ow) and torch.equal(Ls, Lw), case
        Oref, Lref = run_oracle(inp)
        compare(to_np(Os), to_np(Ls), Oref, Lref, f"static scratch {case}")


def test_decode_static_rejects_beyond_scratch():
    # 8 * 32 * 200 rows of 129 floats per split: three splits exceed the scratch
    B, H, Hkv, Sq, Skv, D = 8, 32, 8, 200, 256, 128
    assert fa.flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, 3) > fa._lib.STATIC_SCRATCH_BYTES
    q = torch.zeros(B, H, Sq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Hkv, Skv, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    st = fa.flexattn_decode_static(q, k, k, out, None, B, H, Hkv, Sq, Skv, D, 0.1, 0, 0, None, None, 3,
                                   check=False)
    assert st == fa._lib.ERR_SCRATCH
    assert "static scratch" in fa.flexattn_last_error()
