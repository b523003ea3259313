"""Fused, tiled attention forward for AMD MI355X (gfx950).

The computation runs entirely in the HIP kernels of libflexattn.so; this
package only marshals arguments. `flexattn_*` mirror the C ABI of
include/flexattn.h one to one. `attention()` and `build_block_mask()` are
conveniences that allocate outputs with torch and call those entry points.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from ._lib import (  # noqa: F401
    BF16, FP32, MASK_CAUSAL, MASK_DOCUMENT, MASK_NONE, MASK_PREFIX, MASK_WINDOW, MOD_ALIBI, MOD_NONE,
    MOD_RELBIAS, MOD_SOFTCAP, QTILE, REL_MAX, TILE, BlockMask, FlexAttnError, Params, flexattn_block_mask_bytes,
    flexattn_build_block_mask, flexattn_bwd, flexattn_decode, flexattn_decode_splits,
    flexattn_decode_static, flexattn_decode_workspace_bytes, flexattn_fwd, flexattn_last_error,
    flexattn_split_count,
    flexattn_strerror, flexattn_version, lib,
)

__all__ = [
    "QTILE", "TILE", "flexattn_fwd", "flexattn_bwd", "flexattn_build_block_mask", "flexattn_block_mask_bytes", "flexattn_strerror",
    "flexattn_last_error", "flexattn_version", "attention", "build_block_mask", "make_params",
    "mask_kind_of", "Variant", "BuiltBlockMask", "FlexAttnError", "attention_backward",
    "flexattn_decode", "flexattn_decode_splits", "flexattn_decode_workspace_bytes", "decode",
    "flexattn_split_count", "check_variant", "non_overlapping", "flexattn_decode_static",
]

_DTYPES = {torch.bfloat16: BF16, torch.float32: FP32}


@dataclass
class Variant:
    """A mask_mod / score_mod selection with its parameters (device tensors)."""

    causal: bool = False
    window: int = 0                       # > 0: keep keys with q - k < window
    doc_ids: torch.Tensor | None = None   # int32 [B, >= max(Sq + q_offset, Skv)] on the device
    alibi_slopes: torch.Tensor | None = None  # float32 [H] on the device
    softcap: float | None = None
    q_offset: int = 0                     # query row i sits at key position i + q_offset
    prefix: int | None = None             # with causal: keys below it are seen by every query
    rel_bias: torch.Tensor | None = None  # float32 [H, 2R + 1] on the device: relative-position bias

    @property
    def mask_kind(self) -> int:
        return mask_kind_of(self.causal, self.window, self.doc_ids is not None,
                            self.prefix is not None)

    @property
    def mod_kind(self) -> int:
        if sum(x is not None for x in (self.alibi_slopes, self.softcap, self.rel_bias)) > 1:
            raise ValueError("one score modification at a time")
        if self.rel_bias is not None:
            return MOD_RELBIAS
        if self.alibi_slopes is not None:
            return MOD_ALIBI
        if self.softcap is not None:
            return MOD_SOFTCAP
        return MOD_NONE


def mask_kind_of(causal: bool, window: int, documents: bool, prefix: bool = False) -> int:
    return ((MASK_CAUSAL if causal else 0) | (MASK_WINDOW if window and window > 0 else 0)
            | (MASK_DOCUMENT if documents else 0) | (MASK_PREFIX if prefix else 0))


def set_layout(p: Params, q, k, v, out) -> None:
    """Element strides {batch, head, row} of [B, H, S, D] tensors whose last
    dimension is contiguous (views of other layouts, e.g. [B, S, H, D]
    transposed, need no copy)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out)):
        if t.stride(3) != 1:
            raise TypeError(f"{name}: the last dimension must be contiguous")
        getattr(p, f"{name}_stride")[:] = [t.stride(0), t.stride(1), t.stride(2)]


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _same_device(t: torch.Tensor, device) -> bool:
    device = torch.device(device)
    if t.device.type != device.type:
        return False
    return device.index is None or t.device.index is None or t.device.index == device.index


def check_variant(var: Variant, B: int, H: int | None, Sq: int, Skv: int, device) -> None:
    """Check the variant's device tensors against the call's sizes. The C ABI
    receives them as bare pointers and cannot see their extents, so a short
    tensor would be read past its end on the device; this is the one place
    that can reject it."""
    need_pos = max(Sq + int(var.q_offset), Skv)
    if var.doc_ids is not None:
        d = var.doc_ids
        _need(d.dtype == torch.int32 and d.is_contiguous() and d.dim() == 2,
              "doc_ids must be a contiguous int32 [B, positions] tensor")
        _need(_same_device(d, device), "doc_ids must be on the device of q")
        _need(d.shape[0] >= B, f"doc_ids has {d.shape[0]} rows, the call has B = {B}")
        _need(d.shape[1] >= need_pos,
              f"doc_ids rows hold {d.shape[1]} labels, the call needs {need_pos} (max(Sq + q_offset, Skv))")
    if H is None:
        return
    if var.alibi_slopes is not None:
        a = var.alibi_slopes
        _need(a.dtype == torch.float32 and a.is_contiguous() and a.dim() == 1,
              "alibi_slopes must be a contiguous float32 [H] tensor")
        _need(_same_device(a, device), "alibi_slopes must be on the device of q")
        _need(a.numel() >= H, f"alibi_slopes has {a.numel()} entries, the call has H = {H}")
    if var.rel_bias is not None:
        r = var.rel_bias
        _need(r.dtype == torch.float32 and r.is_contiguous() and r.dim() == 2,
              "rel_bias must be a contiguous float32 [H, 2R + 1] tensor")
        _need(_same_device(r, device), "rel_bias must be on the device of q")
        _need(r.shape[0] >= H, f"rel_bias has {r.shape[0]} rows, the call has H = {H}")
        _need(r.shape[1] % 2 == 1, f"rel_bias rows must hold an odd count 2R + 1, not {r.shape[1]}")


def non_overlapping(t: torch.Tensor) -> bool:
    """True when no two elements of t share an address (ordered by stride,
    every dimension longer than 1 steps over the span of those below it: the
    rule flexattn_bwd applies to the layouts its gradients take)."""
    span = 1
    for stride, size in sorted(zip(t.stride(), t.shape)):
        if size <= 1:
            continue
        if stride < span:
            return False
        span = stride * size
    return True


def make_params(var: Variant, dtype: torch.dtype) -> Params:
    p = Params()
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {dtype}")
    p.dtype = _DTYPES[dtype]
    p.window = int(var.window or 0)
    p.softcap = float(var.softcap) if var.softcap is not None else 0.0
    p.alibi_slopes = var.alibi_slopes.data_ptr() if var.alibi_slopes is not None else None
    p.q_offset = int(var.q_offset)
    if var.rel_bias is not None:
        if var.rel_bias.dtype != torch.float32 or not var.rel_bias.is_contiguous() or var.rel_bias.dim() != 2:
            raise TypeError("rel_bias must be a contiguous float32 [H, 2R + 1] tensor")
        p.rel_bias = var.rel_bias.data_ptr()
        p.rel_max = (int(var.rel_bias.shape[1]) - 1) // 2
    p.prefix = int(var.prefix) if var.prefix is not None else 0
    if var.doc_ids is not None:
        if var.doc_ids.dtype != torch.int32 or not var.doc_ids.is_contiguous():
            raise TypeError("doc_ids must be a contiguous int32 tensor")
        p.doc_ids = var.doc_ids.data_ptr()
        p.doc_stride = int(var.doc_ids.shape[-1])
    return p


@dataclass
class BuiltBlockMask:
    """A block mask and the device buffer that holds its lists."""

    struct: BlockMask
    buf: torch.Tensor

    def counts(self) -> torch.Tensor:
        s = self.struct
        return self.buf[: s.num_b * s.nq].view(s.num_b, s.nq)

    def lists(self) -> torch.Tensor:
        s = self.struct
        return self.buf[s.num_b * s.nq:].view(s.num_b, s.nq, s.nk)


def build_block_mask(var: Variant, B: int, Sq: int, Skv: int, device=None,
                     stream=None) -> BuiltBlockMask:
    """Allocate the list buffer and enqueue flexattn_build_block_mask."""
    mk = var.mask_kind
    nbytes = flexattn_block_mask_bytes(B, Sq, Skv, mk)
    if nbytes == 0:
        raise ValueError("invalid sizes or mask kind for a block mask")
    device = device or (var.doc_ids.device if var.doc_ids is not None else torch.device("cuda"))
    check_variant(var, B, None, Sq, Skv, device)
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
    out = BlockMask()
    flexattn_build_block_mask(mk, make_params(var, torch.bfloat16), B, Sq, Skv, buf, nbytes, out,
                              stream)
    return BuiltBlockMask(out, buf)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, var: Variant | None = None, *,
              scale: float | None = None, block_mask: BuiltBlockMask | None | str = "auto",
              out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
              with_lse: bool = True, stream=None):
    """O (and LSE) of the attention forward for [B, H, S, D] tensors (any
    strides with a contiguous last dimension; `out` defaults to q's layout).

    block_mask: "auto" builds one for the variant; None visits every key tile
    with the per-element mask; or a BuiltBlockMask from build_block_mask().
    """
    var = var or Variant()
    B, H, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    for t in (q, k, v):
        if not t.is_cuda or t.dtype != q.dtype or t.dim() != 4:
            raise TypeError("q, k, v must be 4-D device tensors of one dtype")
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch between q, k and v")
    check_variant(var, B, H, Sq, Skv, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if isinstance(block_mask, str):
        block_mask = build_block_mask(var, B, Sq, Skv, q.device, stream)
    params = make_params(var, q.dtype)
    set_layout(params, q, k, v, out)
    flexattn_fwd(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, scale, var.mask_kind, var.mod_kind,
                 params, block_mask.struct if block_mask is not None else None, stream)
    return out, lse


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, var: Variant | None = None, *,
           scale: float | None = None, block_mask: BuiltBlockMask | None | str = "auto",
           splits: int | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, with_lse: bool = True,
           workspace: torch.Tensor | None = None, stream=None):
    """attention() with the key range split `splits` ways (bf16; default
    flexattn_split_count). With few query rows per key/value head (decoding,
    short prefill chunks) the query heads of a group share a workgroup; with
    more, every 256-row query tile's key list is split, which fills the chip
    when heads are few. The split results need a float32 workspace, allocated
    here unless given."""
    var = var or Variant()
    B, H, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    for t in (q, k, v):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4:
            raise TypeError("q, k, v must be 4-D bf16 device tensors")
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch between q, k and v")
    check_variant(var, B, H, Sq, Skv, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    splits = flexattn_split_count(B, H, Hkv, Sq, Skv) if splits is None else int(splits)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    nbytes = flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    if isinstance(block_mask, str):
        block_mask = build_block_mask(var, B, Sq, Skv, q.device, stream)
    params = make_params(var, q.dtype)
    set_layout(params, q, k, v, out)
    flexattn_decode(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, scale, var.mask_kind, var.mod_kind,
                    params, block_mask.struct if block_mask is not None else None, splits,
                    workspace, workspace.numel() * 4 if workspace is not None else 0, stream)
    return out, lse


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, dout: torch.Tensor, var: Variant | None = None, *,
                       scale: float | None = None,
                       block_mask: BuiltBlockMask | None | str = "auto",
                       dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                       dv: torch.Tensor | None = None, delta: torch.Tensor | None = None,
                       stream=None):
    """(dQ, dK, dV) for the loss sum(out * dout), with out and lse from
    attention() on the same inputs and variant (bf16 tensors). The tensors may
    be strided views (last dimension contiguous), e.g. [B, S, H, D] buffers
    transposed; each gradient has the layout of its input (dq of q, dk of k,
    dv of v, dout of out), and gradients allocated here follow that rule.
    `delta` is the [B, H, Sq] float32 scratch the call needs (allocated here
    if not given)."""
    var = var or Variant()
    B, H, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    for t in (q, k, v, out, dout):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise TypeError("q, k, v, out, dout must be bf16 device tensors")
    if out.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("shape mismatch")
    check_variant(var, B, H, Sq, Skv, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    # Each gradient takes its input's strides. An input whose elements share
    # addresses (e.g. K expanded over the batch) is copied first, so that its
    # gradient gets a layout of its own: the gradient with respect to the
    # view, one slice per batch row or head (a caller that expanded the
    # tensor sums them, as autograd does for expand).
    q, k, v = (t if non_overlapping(t) else t.contiguous() for t in (q, k, v))

    def like(t):
        return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)

    dq = like(q) if dq is None else dq
    dk = like(k) if dk is None else dk
    dv = like(v) if dv is None else dv
    for name, grad, ref in (("dout", dout, out), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if grad.shape != ref.shape or grad.stride() != ref.stride() or grad.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16 with the shape and strides of the tensor it belongs to")
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if isinstance(block_mask, str):
        block_mask = build_block_mask(var, B, Sq, Skv, q.device, stream)
    p = make_params(var, q.dtype)
    if not non_overlapping(out):
        raise ValueError("out must not overlap itself (it is the forward's output)")
    set_layout(p, q, k, v, out)
    flexattn_bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, B, H, Hkv, Sq, Skv, D, scale,
                 var.mask_kind, var.mod_kind, p, block_mask.struct if block_mask is not None else None, stream)
    return dq, dk, dv
