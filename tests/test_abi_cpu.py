"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects invalid calls with the documented status codes before
touching the GPU (validation is pure host code).

These calls pass fake, never-dereferenced addresses, so every case here must
fail validation; they are skipped where a GPU is visible, so that a mistake in
a case can never turn into a launch.
"""
import ctypes
import os
import re

import pytest

import attention_tiled_attn_amd as fa
from attention_tiled_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flexattn.h")


@pytest.fixture(scope="module", autouse=True)
def cpu_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libflexattn.so is not built (python -m attention_tiled_attn_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flexattn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert getattr(L, n) is not None


def test_version_and_strings():
    assert fa.flexattn_version() == 4
    for code in range(-9, 1):
        assert fa.flexattn_strerror(code) and fa.flexattn_strerror(code) != "unknown status"
    assert fa.flexattn_strerror(-99) == "unknown status"
    assert fa.flexattn_last_error() == ""


def test_block_mask_bytes():
    # [num_b][nq] counts + [num_b][nq][nk] lists, nq = ceil(Sq / 256), nk = ceil(Skv / 128)
    assert fa.flexattn_block_mask_bytes(2, 256, 384, 1) == 1 * 1 * (1 + 3) * 4
    assert fa.flexattn_block_mask_bytes(2, 257, 384, 4) == 2 * 2 * (1 + 3) * 4
    assert fa.flexattn_block_mask_bytes(1, 129, 129, 0) == 1 * 3 * 4
    for bad in [(0, 128, 128, 0), (1, 0, 128, 0), (1, 128, -1, 0), (1, 128, 128, 16),
                (1, 128, 128, -1)]:
        assert fa.flexattn_block_mask_bytes(*bad) == 0


A = 0x10000          # 16-byte aligned, never dereferenced
GOOD = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, Hkv=2, Sq=128, Skv=128, D=64, scale=0.125,
            mask_kind=0, mod_kind=0)


def call(**over):
    a = dict(GOOD)
    params = over.pop("params", None)
    bm = over.pop("block_mask", None)
    a.update(over)
    return fa.flexattn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Hkv"],
                           a["Sq"], a["Skv"], a["D"], a["scale"], a["mask_kind"], a["mod_kind"],
                           params, bm, stream=None, check=False)


def P(**kw):
    p = _lib.Params()
    p.dtype = kw.get("dtype", _lib.BF16)
    p.window = kw.get("window", 0)
    p.softcap = kw.get("softcap", 0.0)
    p.alibi_slopes = kw.get("alibi_slopes")
    p.doc_ids = kw.get("doc_ids")
    p.doc_stride = kw.get("doc_stride", 0)
    p.q_offset = kw.get("q_offset", 0)
    p.prefix = kw.get("prefix", 0)
    p.rel_bias = kw.get("rel_bias")
    p.rel_max = kw.get("rel_max", 0)
    for name in ("q", "k", "v", "o"):
        if name + "_stride" in kw:
            getattr(p, name + "_stride")[:] = kw[name + "_stride"]
    return p


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.ERR_NULLPTR),
    (dict(k=None), _lib.ERR_NULLPTR),
    (dict(v=None), _lib.ERR_NULLPTR),
    (dict(out=None), _lib.ERR_NULLPTR),
    (dict(B=0), _lib.ERR_SHAPE),
    (dict(H=0), _lib.ERR_SHAPE),
    (dict(Hkv=0), _lib.ERR_SHAPE),
    (dict(H=3, Hkv=2), _lib.ERR_SHAPE),
    (dict(Sq=0), _lib.ERR_SHAPE),
    (dict(Skv=-5), _lib.ERR_SHAPE),
    (dict(D=96), _lib.ERR_UNSUPPORTED),
    (dict(D=512), _lib.ERR_UNSUPPORTED),
    (dict(D=256, params=P(dtype=_lib.FP32)), _lib.ERR_UNSUPPORTED),   # D = 256 is bf16 only
    (dict(D=256, Skv=2048 * 128 + 1), _lib.ERR_UNSUPPORTED),
    (dict(D=256, out=A + 2), _lib.ERR_ALIGN),                          # bf16 D = 256 is accepted
    (dict(mask_kind=16), _lib.ERR_UNSUPPORTED),
    (dict(mask_kind=8), _lib.ERR_ARG),                                   # prefix without causal
    (dict(mask_kind=10, params=P(window=4)), _lib.ERR_ARG),
    (dict(mask_kind=9, params=P(prefix=-1)), _lib.ERR_ARG),
    (dict(params=P(q_offset=-1)), _lib.ERR_ARG),
    (dict(mask_kind=1, params=P(q_offset=2**31 - 300)), _lib.ERR_OVERFLOW),
    (dict(mask_kind=4, params=P(doc_ids=A, doc_stride=128, q_offset=1)), _lib.ERR_ARG),  # stride < Sq + off
    (dict(mask_kind=-1), _lib.ERR_UNSUPPORTED),
    (dict(mod_kind=4), _lib.ERR_UNSUPPORTED),
    (dict(mod_kind=3, params=P()), _lib.ERR_NULLPTR),                     # relative bias, no table
    (dict(mod_kind=3, params=P(rel_bias=A + 4)), _lib.ERR_ALIGN),
    (dict(mod_kind=3, params=P(rel_bias=A, rel_max=-1)), _lib.ERR_ARG),
    (dict(mod_kind=3, params=P(rel_bias=A, rel_max=1024)), _lib.ERR_ARG),
    (dict(params=P(dtype=7)), _lib.ERR_UNSUPPORTED),
    (dict(scale=float("nan")), _lib.ERR_ARG),
    (dict(scale=float("inf")), _lib.ERR_ARG),
    (dict(scale=0.0), _lib.ERR_ARG),
    (dict(scale=-0.5), _lib.ERR_ARG),
    (dict(Sq=5_000_000, D=128, params=P(dtype=_lib.FP32)), _lib.ERR_OVERFLOW),
    (dict(q=A + 8), _lib.ERR_ALIGN),
    (dict(out=A + 2), _lib.ERR_ALIGN),
    (dict(lse=A + 2), _lib.ERR_ALIGN),
    (dict(mask_kind=2, params=P(window=0)), _lib.ERR_ARG),
    (dict(mask_kind=3), _lib.ERR_ARG),                                   # window with no params
    (dict(mask_kind=4, params=P()), _lib.ERR_NULLPTR),                   # documents, no labels
    (dict(mask_kind=4, params=P(doc_ids=A, doc_stride=100)), _lib.ERR_ARG),  # stride < S
    (dict(mask_kind=4, params=P(doc_ids=A + 2, doc_stride=128)), _lib.ERR_ALIGN),
    (dict(mask_kind=4, params=P(doc_ids=A, doc_stride=2**29)), _lib.ERR_OVERFLOW),   # byte offsets past 2^31
    (dict(mod_kind=1, params=P()), _lib.ERR_NULLPTR),                    # ALiBi, no slopes
    (dict(mod_kind=1, params=P(alibi_slopes=A + 1)), _lib.ERR_ALIGN),
    (dict(mod_kind=2, params=P(softcap=0.0)), _lib.ERR_ARG),
    (dict(mod_kind=2, params=P(softcap=-3.0)), _lib.ERR_ARG),
    (dict(mod_kind=2, params=P(softcap=float("inf"))), _lib.ERR_ARG),
    (dict(Sq=2**31 - 100), _lib.ERR_OVERFLOW),
    (dict(B=2**20, H=2**12, Hkv=1, Sq=256), _lib.ERR_OVERFLOW),
])
def test_fwd_validation(over, code):
    assert call(**over) == code


# layouts: GOOD is B=1, H=2, S=128, D=64 in bf16 (16 bytes = 8 elements)
@pytest.mark.parametrize("stride,code", [
    ((64 * 128, 64, 64 * 2), _lib.ERR_ALIGN),       # ok up to here? see below
    ((2 * 128 * 64, 128 * 64, 63), _lib.ERR_ARG),    # row stride below D
    ((2 * 128 * 64, 128 * 64, 68), _lib.ERR_ALIGN),  # rows not 16-byte aligned
    ((-8, 128 * 64, 64), _lib.ERR_ARG),              # negative
    ((2 * 128 * 64, 4, 64), _lib.ERR_ALIGN),         # head stride not 16-byte aligned
    ((0, 0, 2**26), _lib.ERR_OVERFLOW),              # a slice beyond 32-bit byte offsets
])
@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_fwd_layout_validation(stride, code, which):
    if stride == (64 * 128, 64, 64 * 2):
        # a valid [B, S, H, D] view: stops at the misaligned output instead
        assert call(params=P(**{which + "_stride": stride}), out=A + 2) == _lib.ERR_ALIGN
        return
    assert call(params=P(**{which + "_stride": stride})) == code


def bm_struct(**kw):
    s = _lib.BlockMask()
    s.tile_q = kw.get("tile_q", 256)
    s.tile_k = kw.get("tile_k", 128)
    s.nq = kw.get("nq", 1)
    s.nk = kw.get("nk", 1)
    s.num_b = kw.get("num_b", 1)
    s.mask_kind = kw.get("mask_kind", 0)
    s.Sq = kw.get("Sq", 128)
    s.Skv = kw.get("Skv", 128)
    s.kv_count = kw.get("kv_count", A)
    s.kv_list = kw.get("kv_list", A)
    s.window = kw.get("window", 0)
    s.q_offset = kw.get("q_offset", 0)
    s.prefix = kw.get("prefix", 0)
    return s


@pytest.mark.parametrize("kw", [
    dict(tile_q=128), dict(tile_k=256), dict(nq=2), dict(nk=3), dict(mask_kind=1), dict(Sq=127),
    dict(Skv=100), dict(num_b=2), dict(kv_count=None), dict(kv_list=None),
])
def test_fwd_rejects_mismatched_block_mask(kw):
    assert call(block_mask=bm_struct(**kw)) == _lib.ERR_BLOCKMASK


@pytest.mark.parametrize("mk,params,kw,code", [
    # the parameters a block mask was built with must match where the mask uses them
    (3, dict(window=64), dict(window=64), _lib.OK),
    (3, dict(window=64), dict(window=65), _lib.ERR_BLOCKMASK),
    (1, dict(q_offset=5), dict(q_offset=5), _lib.OK),
    (1, dict(q_offset=5), dict(), _lib.ERR_BLOCKMASK),
    (9, dict(prefix=40), dict(prefix=40), _lib.OK),
    (9, dict(prefix=40), dict(prefix=41), _lib.ERR_BLOCKMASK),
    (1, dict(prefix=40), dict(), _lib.OK),            # no PREFIX bit: prefix unused
    (0, dict(q_offset=5, window=3), dict(), _lib.OK),  # no mask: nothing positional
])
def test_block_mask_records_its_params(mk, params, kw, code):
    bm = bm_struct(mask_kind=mk, **kw)
    if code == _lib.OK:
        # a matching mask passes validation; the misaligned output, checked
        # after the mask, stops the call before any launch
        assert call(mask_kind=mk, params=P(**params), block_mask=bm, out=A + 2) == _lib.ERR_ALIGN
    else:
        assert call(mask_kind=mk, params=P(**params), block_mask=bm) == code


def test_build_block_mask_validation():
    out = _lib.BlockMask()

    def b(mk, params, B, Sq, Skv, buf, nbytes):
        return fa.flexattn_build_block_mask(mk, params, B, Sq, Skv, buf, nbytes, out, None,
                                            check=False)
    need = fa.flexattn_block_mask_bytes(1, 256, 256, 1)
    assert b(1, None, 1, 256, 256, None, need) == _lib.ERR_NULLPTR
    assert b(1, None, 1, 256, 256, A + 2, need) == _lib.ERR_ALIGN
    assert b(1, None, 1, 256, 256, A, need - 4) == _lib.ERR_ARG
    assert b(17, None, 1, 256, 256, A, need) == _lib.ERR_UNSUPPORTED
    assert b(8, None, 1, 256, 256, A, need) == _lib.ERR_ARG          # prefix needs causal
    assert b(1, P(q_offset=-3), 1, 256, 256, A, need) == _lib.ERR_ARG
    assert b(1, None, 0, 256, 256, A, need) == _lib.ERR_SHAPE
    assert b(2, None, 1, 256, 256, A, need) == _lib.ERR_ARG          # window needs params
    assert b(4, P(), 1, 256, 256, A, need) == _lib.ERR_NULLPTR        # documents need labels
    L = _lib.lib()
    assert L.flexattn_build_block_mask(1, None, 1, 256, 256, A, need, None, None) == _lib.ERR_NULLPTR


def test_error_raises_with_message():
    with pytest.raises(fa.FlexAttnError, match="invalid shape"):
        fa.flexattn_fwd(A, A, A, A, A, 0, 2, 2, 128, 128, 64, 0.1, 0, 0)


# ------------------------------------------------------------------ backward validation
BGOOD = dict(q=A, k=A, v=A, out=A, lse=A, dout=A, dq=A, dk=A, dv=A, delta=A, B=1, H=2, Hkv=2,
             Sq=128, Skv=128, D=64, scale=0.125, mask_kind=0, mod_kind=0)


@pytest.mark.parametrize("stride,code", [
    ((64 * 128, 64, 64 * 2), _lib.ERR_ALIGN),       # a valid [B, S, H, D] view; see below
    ((2 * 128 * 64, 128 * 64, 63), _lib.ERR_ARG),    # row stride below D
    ((2 * 128 * 64, 128 * 64, 68), _lib.ERR_ALIGN),  # rows not 16-byte aligned
    ((-8, 128 * 64, 64), _lib.ERR_ARG),              # negative
    ((0, 0, 2**26), _lib.ERR_OVERFLOW),              # a slice beyond 32-bit byte offsets
])
@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_bwd_layout_validation(stride, code, which):
    # the backward takes the forward's layouts (gradients share their input's strides)
    if stride == (64 * 128, 64, 64 * 2):
        assert bcall(params=P(**{which + "_stride": stride}), dq=A + 2) == _lib.ERR_ALIGN
        return
    assert bcall(params=P(**{which + "_stride": stride})) == code


def bcall(**over):
    a = dict(BGOOD)
    params = over.pop("params", None)
    bm = over.pop("block_mask", None)
    a.update(over)
    return fa.flexattn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"],
                           a["dv"], a["delta"], a["B"], a["H"], a["Hkv"], a["Sq"], a["Skv"], a["D"],
                           a["scale"], a["mask_kind"], a["mod_kind"], params, bm, stream=None,
                           check=False)


@pytest.mark.parametrize("over,code", [
    *[(dict(**{name: None}), _lib.ERR_NULLPTR)
      for name in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "delta")],
    (dict(H=3, Hkv=2), _lib.ERR_SHAPE),
    (dict(D=96), _lib.ERR_UNSUPPORTED),
    (dict(params=P(dtype=_lib.FP32)), _lib.ERR_UNSUPPORTED),     # bf16 only
    (dict(Skv=2048 * 128 + 1), _lib.ERR_UNSUPPORTED),           # key-tile list limit
    (dict(scale=0.0), _lib.ERR_ARG),
    (dict(dout=A + 8), _lib.ERR_ALIGN),
    (dict(dq=A + 4), _lib.ERR_ALIGN),
    (dict(dk=A + 2), _lib.ERR_ALIGN),
    (dict(dv=A + 8), _lib.ERR_ALIGN),
    (dict(delta=A + 2), _lib.ERR_ALIGN),
    (dict(lse=A + 1), _lib.ERR_ALIGN),
    (dict(mask_kind=4, params=P()), _lib.ERR_NULLPTR),
    (dict(mod_kind=1, params=P()), _lib.ERR_NULLPTR),
    (dict(block_mask=bm_struct(tile_q=128)), _lib.ERR_BLOCKMASK),
])
def test_bwd_validation(over, code):
    assert bcall(**over) == code


# ------------------------------------------------------------------ decode entry points
def test_decode_workspace_and_splits():
    # splits x rows x (D + 1) floats, rows = B * H * Sq; none for one split
    assert fa.flexattn_decode_workspace_bytes(2, 8, 2, 3, 128, 5) == 5 * (2 * 8 * 3) * 129 * 4
    assert fa.flexattn_decode_workspace_bytes(2, 8, 2, 3, 128, 1) == 0
    for bad in [(0, 8, 2, 1, 128, 2), (1, 8, 3, 1, 128, 2), (1, 8, 2, 1, 96, 2), (1, 8, 2, 1, 64, 65)]:
        assert fa.flexattn_decode_workspace_bytes(*bad) == 0
    # rounds of 256 workgroups x (2 tiles / s + 3) stage times, minimised;
    # at least 4 key tiles each, at most 64
    assert fa.flexattn_decode_splits(16, 8, 32768) == 2       # 128 groups: one round of 256
    assert fa.flexattn_decode_splits(100, 1, 65536) == 5      # 500 workgroups in 2 rounds
    assert fa.flexattn_decode_splits(3, 1, 65536) == 64
    assert fa.flexattn_decode_splits(1, 1, 1 << 20) == 64
    assert fa.flexattn_decode_splits(1, 8, 1024) == 2
    assert fa.flexattn_decode_splits(64, 8, 8192) == 1
    # either organisation: packed decoding takes the rule above; otherwise
    # ~2 workgroups per CU over B * H * ceil(Sq / 256) items, >= 8 key tiles per split
    assert fa.flexattn_split_count(16, 32, 8, 1, 32768) == fa.flexattn_decode_splits(16, 8, 32768)
    assert fa.flexattn_split_count(2, 4, 1, 8192, 8192) == 2      # 256 items
    assert fa.flexattn_split_count(4, 16, 16, 4096, 4096) == 1    # 1024 items
    assert fa.flexattn_split_count(1, 4, 4, 4096, 4096) == 4      # 64 items, 32 key tiles
    assert fa.flexattn_split_count(1, 1, 1, 300, 300) == 1        # 3 key tiles
    assert fa.flexattn_split_count(1, 3, 2, 300, 300) == 1        # invalid: H % Hkv


def dcall(**over):
    a = dict(GOOD, H=8, Hkv=2, Sq=1, Skv=512)
    params = over.pop("params", None)
    splits = over.pop("splits", 2)
    ws = over.pop("ws", A)
    wsb = over.pop("wsb", 1 << 20)
    a.update(over)
    return fa.flexattn_decode(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Hkv"],
                              a["Sq"], a["Skv"], a["D"], a["scale"], a["mask_kind"], a["mod_kind"],
                              params, None, splits, ws, wsb, stream=None, check=False)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.ERR_NULLPTR),
    (dict(params=P(dtype=_lib.FP32)), _lib.ERR_UNSUPPORTED),     # bf16 only
    (dict(Sq=65, H=8, Hkv=2, ws=A + 4), _lib.ERR_ALIGN),        # 4 x 65 rows > 256: split tiles, still checked
    (dict(Sq=65, H=8, Hkv=2, wsb=100), _lib.ERR_ARG),
    (dict(Sq=300, mod_kind=3, params=P(rel_bias=A, rel_max=300), ws=A + 4), _lib.ERR_ALIGN),  # not packed: one table
    (dict(splits=0), _lib.ERR_ARG),
    (dict(splits=65), _lib.ERR_ARG),
    (dict(ws=None), _lib.ERR_NULLPTR),                           # two splits need a workspace
    (dict(ws=A + 4), _lib.ERR_ALIGN),
    (dict(wsb=100), _lib.ERR_ARG),                               # too small
    (dict(mod_kind=3, params=P(rel_bias=A, rel_max=300)), _lib.ERR_UNSUPPORTED),  # 4 tables of 601 > LDS
    (dict(splits=1, ws=None, out=A + 2), _lib.ERR_ALIGN),        # one split needs none: reaches the checks after
])
def test_decode_validation(over, code):
    assert dcall(**over) == code


# ------------------------------------------------------------------ overlapping layouts
# GOOD / BGOOD are B=1, H=2 (Hkv=2), S=128, D=64: contiguous head stride 128*64.
@pytest.mark.parametrize("which,stride,B,code", [
    ("k", (0, 128 * 64, 64), 2, _lib.ERR_ARG),          # K expanded over the batch: dK rows collide
    ("v", (0, 128 * 64, 64), 2, _lib.ERR_ARG),
    ("q", (0, 128 * 64, 64), 2, _lib.ERR_ARG),
    ("k", (2 * 128 * 64, 0, 64), 1, _lib.ERR_ARG),      # heads share one slice
    ("q", (2 * 128 * 64, 64, 64), 1, _lib.ERR_ARG),     # head stride inside a row span
    ("o", (2 * 128 * 64, 0, 64), 1, _lib.ERR_ARG),      # out (and dout) overlapping
    ("k", (0, 128 * 64, 64), 1, _lib.ERR_ALIGN),        # stride 0 over B = 1 is no overlap
    ("k", (64 * 128, 64, 64 * 2), 1, _lib.ERR_ALIGN),   # [B, S, H, D] view: distinct elements
])
def test_bwd_rejects_overlapping_layouts(which, stride, B, code):
    # the calls that pass the overlap rule stop at the misaligned dq after it
    assert bcall(B=B, params=P(**{which + "_stride": stride}), dq=A + 2) == code


@pytest.mark.parametrize("which,stride,code", [
    ("o", (2 * 128 * 64, 0, 64), _lib.ERR_ARG),     # two heads written to one slice
    ("o", (2 * 128 * 64, 128 * 64, 0), _lib.ERR_ARG),   # row stride below D
    ("q", (2 * 128 * 64, 0, 64), _lib.ERR_ALIGN),   # inputs may overlap: read only
    ("k", (0, 0, 64), _lib.ERR_ALIGN),
])
def test_fwd_overlap_rule_applies_to_out_only(which, stride, code):
    assert call(params=P(**{which + "_stride": stride}), lse=A + 2) == code
    assert dcall(params=P(**{which + "_stride": stride}), lse=A + 2) == code


# ------------------------------------------------------------------ allocation-free decode
def scall(**over):
    a = dict(GOOD, H=8, Hkv=2, Sq=1, Skv=512)
    params = over.pop("params", None)
    splits = over.pop("splits", 2)
    a.update(over)
    return fa.flexattn_decode_static(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Hkv"],
                                     a["Sq"], a["Skv"], a["D"], a["scale"], a["mask_kind"], a["mod_kind"],
                                     params, None, splits, stream=None, check=False)


def test_decode_static_validation():
    # the same checks as flexattn_decode, no workspace arguments
    assert scall(q=None) == _lib.ERR_NULLPTR
    assert scall(splits=0) == _lib.ERR_ARG
    assert scall(splits=65) == _lib.ERR_ARG
    assert scall(params=P(dtype=_lib.FP32)) == _lib.ERR_UNSUPPORTED
    assert scall(out=A + 2) == _lib.ERR_ALIGN
    # split results beyond the static scratch: rejected before any HIP call,
    # with the sizes in the message
    B, H, Sq, D = 8, 32, 200, 128        # 8 * 32 * 200 rows * 129 floats = 26.4 MB per split
    need = fa.flexattn_decode_workspace_bytes(B, H, 8, Sq, D, 3)
    assert need > _lib.STATIC_SCRATCH_BYTES >= fa.flexattn_decode_workspace_bytes(B, H, 8, Sq, D, 2)
    assert scall(B=B, H=H, Hkv=8, Sq=Sq, D=D, splits=3) == _lib.ERR_SCRATCH
    assert str(need) in fa.flexattn_last_error() and str(_lib.STATIC_SCRATCH_BYTES) in fa.flexattn_last_error()
    # two splits fit: validation passes, and the misaligned output stops the call
    assert scall(B=B, H=H, Hkv=8, Sq=Sq, D=D, splits=2, out=A + 2) == _lib.ERR_ALIGN
