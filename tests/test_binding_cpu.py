"""The Python binding's own checks, on CPU tensors: the variant's tensors are
passed to the C ABI as bare device pointers, whose extents the library cannot
see, so the binding rejects short or mistyped ones before any call."""
import pytest
import torch

import attention_tiled_attn_amd as fa

B, H, Sq, Skv = 2, 4, 300, 300
CPU = torch.device("cpu")


def ok(**kw):
    fa.check_variant(fa.Variant(**kw), B, H, Sq, Skv, CPU)


def bad(match, **kw):
    with pytest.raises(ValueError, match=match):
        fa.check_variant(fa.Variant(**kw), B, H, Sq, Skv, CPU)


def test_valid_variants_pass():
    ok()
    ok(causal=True, doc_ids=torch.zeros(B, Skv, dtype=torch.int32))
    ok(doc_ids=torch.zeros(B + 1, Skv + 7, dtype=torch.int32), q_offset=7)
    ok(alibi_slopes=torch.ones(H))
    ok(rel_bias=torch.zeros(H, 11))
    # the block-mask builder has no H: only the labels are checked
    fa.check_variant(fa.Variant(alibi_slopes=torch.ones(1)), B, None, Sq, Skv, CPU)


def test_document_labels():
    bad("int32", doc_ids=torch.zeros(B, Skv, dtype=torch.int64))
    bad("int32", doc_ids=torch.zeros(B * Skv, dtype=torch.int32))           # 1-D
    bad("int32", doc_ids=torch.zeros(Skv, B, dtype=torch.int32).t())        # not contiguous
    bad("rows", doc_ids=torch.zeros(B - 1, Skv, dtype=torch.int32))
    bad("labels", doc_ids=torch.zeros(B, Skv - 1, dtype=torch.int32))
    bad("labels", doc_ids=torch.zeros(B, Skv, dtype=torch.int32), q_offset=1)   # Sq + q_offset > Skv


def test_alibi_slopes():
    bad("entries", alibi_slopes=torch.ones(H - 1))
    bad("float32", alibi_slopes=torch.ones(H, dtype=torch.float64))
    bad("float32", alibi_slopes=torch.ones(H, 1))
    bad("float32", alibi_slopes=torch.ones(2 * H)[::2])


def test_relative_bias_table():
    bad("rows", rel_bias=torch.zeros(H - 1, 11))
    bad("odd", rel_bias=torch.zeros(H, 10))
    bad("float32", rel_bias=torch.zeros(H, 11, dtype=torch.float16))
    bad("float32", rel_bias=torch.zeros(H * 11))


def test_device_must_match():
    meta = torch.device("meta")
    with pytest.raises(ValueError, match="device"):
        fa.check_variant(fa.Variant(alibi_slopes=torch.ones(H)), B, H, Sq, Skv, meta)


@pytest.mark.parametrize("t,want", [
    (torch.empty(2, 3, 5, 8), True),
    (torch.empty(2, 5, 3, 8).transpose(1, 2), True),           # [B, S, H, D] viewed
    (torch.empty(1, 3, 5, 8).expand(2, -1, -1, -1), False),    # batch stride 0
    (torch.empty(2, 1, 5, 8).expand(-1, 3, -1, -1), False),    # head stride 0
    (torch.empty(1, 1, 5, 8).expand(1, 1, -1, -1), True),      # stride 0 over extent 1 only
    (torch.empty(2, 3, 6, 8)[:, :, ::2], True),                # row-padded
    (torch.empty(100).as_strided((2, 3, 5, 8), (8, 8, 8, 1)), False),
])
def test_non_overlapping(t, want):
    assert fa.non_overlapping(t) is want
