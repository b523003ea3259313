"""ctypes binding of libflexattn.so: the C ABI of include/flexattn.h under the
same names, with argument marshalling only (tensors -> device pointers, the
current torch stream -> hipStream_t, status codes -> exceptions).

torch is imported before the library is loaded so that the process has one HIP
runtime: the library's dependency on the HIP runtime resolves to the copy torch
already loaded.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the library, see above)

# FLEXATTN_LIB names another build of the same ABI (the sanitizer build of
# the argument checks, loaded by tests/test_abi_sanitized.py)
LIB_PATH = os.environ.get("FLEXATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libflexattn.so")

# status codes and enums, as in include/flexattn.h
OK = 0
ERR_NULLPTR, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN = -1, -2, -3, -4
ERR_BLOCKMASK, ERR_OVERFLOW, ERR_HIP, ERR_ARG = -5, -6, -7, -8
ERR_SCRATCH = -9
STATIC_SCRATCH_BYTES = 64 << 20
BF16, FP32 = 0, 1
MASK_NONE, MASK_CAUSAL, MASK_WINDOW, MASK_DOCUMENT, MASK_PREFIX = 0, 1, 2, 4, 8
MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_RELBIAS = 0, 1, 2, 3
REL_MAX = 1023
TILE = 128
QTILE = 256

EXPORTS = ("flexattn_version", "flexattn_strerror", "flexattn_last_error",
           "flexattn_block_mask_bytes", "flexattn_build_block_mask", "flexattn_fwd", "flexattn_bwd",
           "flexattn_decode_workspace_bytes", "flexattn_decode_splits", "flexattn_split_count",
           "flexattn_decode", "flexattn_decode_static")


class FlexAttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: {flexattn_strerror(status)} ({status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


class Params(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("window", ctypes.c_int), ("softcap", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p), ("doc_ids", ctypes.c_void_p),
                ("doc_stride", ctypes.c_int), ("q_offset", ctypes.c_int), ("prefix", ctypes.c_int),
                ("rel_bias", ctypes.c_void_p), ("rel_max", ctypes.c_int),
                ("q_stride", ctypes.c_longlong * 3), ("k_stride", ctypes.c_longlong * 3),
                ("v_stride", ctypes.c_longlong * 3), ("o_stride", ctypes.c_longlong * 3)]


class BlockMask(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int), ("tile_k", ctypes.c_int), ("nq", ctypes.c_int),
                ("nk", ctypes.c_int), ("num_b", ctypes.c_int), ("mask_kind", ctypes.c_int),
                ("Sq", ctypes.c_int), ("Skv", ctypes.c_int),
                ("kv_count", ctypes.c_void_p), ("kv_list", ctypes.c_void_p),
                ("window", ctypes.c_int), ("q_offset", ctypes.c_int), ("prefix", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_tiled_attn_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_float, vp, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        L.flexattn_version.restype = c_int
        L.flexattn_version.argtypes = []
        L.flexattn_strerror.restype = ctypes.c_char_p
        L.flexattn_strerror.argtypes = [c_int]
        L.flexattn_last_error.restype = ctypes.c_char_p
        L.flexattn_last_error.argtypes = []
        L.flexattn_block_mask_bytes.restype = sz
        L.flexattn_block_mask_bytes.argtypes = [c_int, c_int, c_int, c_int]
        L.flexattn_build_block_mask.restype = c_int
        L.flexattn_build_block_mask.argtypes = [c_int, ctypes.POINTER(Params), c_int, c_int, c_int,
                                                vp, sz, ctypes.POINTER(BlockMask), vp]
        L.flexattn_fwd.restype = c_int
        L.flexattn_fwd.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_float, c_int, c_int, ctypes.POINTER(Params),
                                   ctypes.POINTER(BlockMask), vp]
        L.flexattn_decode_workspace_bytes.restype = sz
        L.flexattn_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
        L.flexattn_decode_splits.restype = c_int
        L.flexattn_decode_splits.argtypes = [c_int, c_int, c_int]
        L.flexattn_split_count.restype = c_int
        L.flexattn_split_count.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.flexattn_decode.restype = c_int
        L.flexattn_decode.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_float, c_int, c_int, ctypes.POINTER(Params),
                                      ctypes.POINTER(BlockMask), c_int, vp, sz, vp]
        L.flexattn_decode_static.restype = c_int
        L.flexattn_decode_static.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                             c_float, c_int, c_int, ctypes.POINTER(Params),
                                             ctypes.POINTER(BlockMask), c_int, vp]
        L.flexattn_bwd.restype = c_int
        L.flexattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int, c_int, c_int,
                                   c_int, c_int, c_int, c_float, c_int, c_int,
                                   ctypes.POINTER(Params), ctypes.POINTER(BlockMask), vp]
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, anchor=None) -> int | None:
    """hipStream_t for a call: an explicit stream (int handle or torch stream),
    else torch's current stream on the anchor tensor's device, else NULL."""
    if stream is None:
        if isinstance(anchor, torch.Tensor) and anchor.is_cuda:
            return torch.cuda.current_stream(anchor.device).cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != OK:
        detail = flexattn_last_error() if status == ERR_HIP else ""
        raise FlexAttnError(status, where, detail)


# ------------------------------------------------------------------ the C ABI, same names
def flexattn_version() -> int:
    return lib().flexattn_version()


def flexattn_strerror(status: int) -> str:
    return lib().flexattn_strerror(status).decode()


def flexattn_last_error() -> str:
    return lib().flexattn_last_error().decode()


def flexattn_block_mask_bytes(B: int, Sq: int, Skv: int, mask_kind: int) -> int:
    return int(lib().flexattn_block_mask_bytes(B, Sq, Skv, mask_kind))


def flexattn_build_block_mask(mask_kind: int, params: Params | None, B: int, Sq: int, Skv: int,
                              buf, nbytes: int, out: BlockMask, stream=None, *,
                              check: bool = True) -> int:
    st = lib().flexattn_build_block_mask(mask_kind, ctypes.byref(params) if params else None,
                                         B, Sq, Skv, _ptr(buf), nbytes, ctypes.byref(out),
                                         _stream(stream, buf))
    if check:
        _check(st, "flexattn_build_block_mask")
    return st


def flexattn_fwd(q, k, v, out, lse, B: int, H: int, Hkv: int, Sq: int, Skv: int, D: int,
                 scale: float, mask_kind: int, mod_kind: int, params: Params | None = None,
                 block_mask: BlockMask | None = None, stream=None, *, check: bool = True) -> int:
    st = lib().flexattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Sq, Skv,
                            D, scale, mask_kind, mod_kind,
                            ctypes.byref(params) if params else None,
                            ctypes.byref(block_mask) if block_mask else None,
                            _stream(stream, q))
    if check:
        _check(st, "flexattn_fwd")
    return st


def flexattn_decode_workspace_bytes(B: int, H: int, Hkv: int, Sq: int, D: int, splits: int) -> int:
    return int(lib().flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits))


def flexattn_decode_splits(B: int, Hkv: int, Skv: int) -> int:
    return int(lib().flexattn_decode_splits(B, Hkv, Skv))


def flexattn_split_count(B: int, H: int, Hkv: int, Sq: int, Skv: int) -> int:
    return int(lib().flexattn_split_count(B, H, Hkv, Sq, Skv))


def flexattn_decode(q, k, v, out, lse, B: int, H: int, Hkv: int, Sq: int, Skv: int, D: int,
                    scale: float, mask_kind: int, mod_kind: int, params: Params | None = None,
                    block_mask: BlockMask | None = None, splits: int = 1, workspace=None,
                    workspace_bytes: int = 0, stream=None, *, check: bool = True) -> int:
    st = lib().flexattn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Sq, Skv,
                               D, scale, mask_kind, mod_kind,
                               ctypes.byref(params) if params else None,
                               ctypes.byref(block_mask) if block_mask else None, splits,
                               _ptr(workspace), workspace_bytes, _stream(stream, q))
    if check:
        _check(st, "flexattn_decode")
    return st


def flexattn_decode_static(q, k, v, out, lse, B: int, H: int, Hkv: int, Sq: int, Skv: int, D: int,
                           scale: float, mask_kind: int, mod_kind: int, params: Params | None = None,
                           block_mask: BlockMask | None = None, splits: int = 1, stream=None, *,
                           check: bool = True) -> int:
    st = lib().flexattn_decode_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Sq,
                                      Skv, D, scale, mask_kind, mod_kind,
                                      ctypes.byref(params) if params else None,
                                      ctypes.byref(block_mask) if block_mask else None, splits,
                                      _stream(stream, q))
    if check:
        _check(st, "flexattn_decode_static")
    return st


def flexattn_bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, B: int, H: int, Hkv: int, Sq: int,
                 Skv: int, D: int, scale: float, mask_kind: int, mod_kind: int,
                 params: Params | None = None, block_mask: BlockMask | None = None, stream=None, *,
                 check: bool = True) -> int:
    st = lib().flexattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                            _ptr(dk), _ptr(dv), _ptr(delta), B, H, Hkv, Sq, Skv, D, scale,
                            mask_kind, mod_kind, ctypes.byref(params) if params else None,
                            ctypes.byref(block_mask) if block_mask else None, _stream(stream, q))
    if check:
        _check(st, "flexattn_bwd")
    return st
