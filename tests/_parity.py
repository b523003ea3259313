"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the binding, run the oracle on the values the GPU
consumed, and compare at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import attention_tiled_attn_amd as fa
import oracle
from workload import Inputs, Workload, bf16_values, make_inputs

# Tolerances: bf16 output against the fp64 oracle.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def pair_lists(ref: np.ndarray) -> list[list[int]]:
    """Expected block-mask lists from per-(128-row tile, 128-key tile) classes
    (0 empty, 1 partial, 2 full): one list per 256-row query tile, entry
    (kv_tile << 4) | class bits of half 1 << 2 | class bits of half 0, where a
    class is coded 0 (empty), 1 (partial) or 3 (full)."""
    code = {0: 0, 1: 1, 2: 3}
    out = []
    for qp in range((ref.shape[0] + 1) // 2):
        lst = []
        for j in range(ref.shape[1]):
            bits = code[int(ref[2 * qp, j])]
            if 2 * qp + 1 < ref.shape[0]:
                bits |= code[int(ref[2 * qp + 1, j])] << 2
            if bits:
                lst.append((j << 4) | bits)
        out.append(lst)
    return out


def check_pair_lists(counts: np.ndarray, lists: np.ndarray, ref: np.ndarray) -> None:
    """Assert that the block-mask lists of one batch row equal the lists that
    per-(128-row tile, 128-key tile) classes `ref` (0 empty, 1 partial, 2
    full; from the oracle's pair-by-pair test) give: every key tile, its
    order and both halves' classes, bit for bit (index work is exact)."""
    for qp, want in enumerate(pair_lists(ref)):
        got = lists[qp, :counts[qp]].tolist()
        assert got == want, (qp, [e for e in got if e not in want][:8], [e for e in want if e not in got][:8])


def device_variant(inp: Inputs, device="cuda") -> fa.Variant:
    wl = inp.wl
    return fa.Variant(
        causal=wl.causal,
        window=wl.window,
        doc_ids=torch.from_numpy(inp.doc_ids).to(device) if inp.doc_ids is not None else None,
        alibi_slopes=torch.from_numpy(inp.slopes).to(device) if inp.slopes is not None else None,
        softcap=wl.softcap if wl.mod == "softcap" else None,
        q_offset=wl.q_offset,
        prefix=wl.prefix,
        rel_bias=torch.from_numpy(inp.rel_bias).to(device) if inp.rel_bias is not None else None,
    )


def run_gpu(inp: Inputs, block_mask="auto", var=None, qkv=None):
    """(O, LSE) device tensors from the HIP path."""
    q, k, v = qkv if qkv is not None else (t.cuda() for t in (inp.q, inp.k, inp.v))
    var = var or device_variant(inp)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.attention(q, k, v, var, scale=inp.wl.scale, block_mask=block_mask, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_kwargs(inp: Inputs) -> dict:
    wl = inp.wl
    return dict(causal=wl.causal, window=wl.window or None, doc_ids=inp.doc_ids,
                alibi_slopes=None if inp.slopes is None else inp.slopes.astype(np.float64),
                softcap=wl.softcap if wl.mod == "softcap" else None, q_offset=wl.q_offset,
                prefix=wl.prefix,
                rel_bias=None if inp.rel_bias is None else inp.rel_bias.astype(np.float64))


def run_oracle(inp: Inputs, rows=None, heads=None):
    """Oracle on exactly the values the GPU consumes (bf16; fp32 inputs are
    rounded to bf16 on load by the kernel)."""
    q, k, v = (bf16_values(t) for t in (inp.q, inp.k, inp.v))
    return oracle.attention(q, k, v, inp.wl.scale, rows=rows, heads=heads, **oracle_kwargs(inp))


def run_oracle_full(inp: Inputs, heads=None, stats=None):
    """The oracle over whole tensors (every batch row, head and query row
    unless `heads` is given), in a pool of host processes."""
    from oracle.pool import attention_parallel
    q, k, v = (bf16_values(t) for t in (inp.q, inp.k, inp.v))
    return attention_parallel(q, k, v, inp.wl.scale, heads=heads, stats=stats, **oracle_kwargs(inp))


def compare(O, L, Oref, Lref, what=""):
    """Assert the GPU result (numpy float64) matches the oracle."""
    assert not np.isnan(O).any(), f"{what}: NaN in O"
    assert not np.isnan(L).any(), f"{what}: NaN in LSE"
    ninf = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), ninf), f"{what}: -inf rows differ"
    if ninf.any():
        assert (O[ninf] == 0).all(), f"{what}: fully masked rows must be zero"
    err = np.abs(O - Oref)
    lerr = np.abs(L[~ninf] - Lref[~ninf])
    stats = dict(max_abs=float(err.max(initial=0)), mean_abs=float(err.mean()) if err.size else 0.0,
                 lse_max=float(lerr.max(initial=0)))
    assert stats["max_abs"] <= O_MAX_ABS, f"{what}: {stats}"
    assert stats["mean_abs"] <= O_MEAN_ABS, f"{what}: {stats}"
    assert stats["lse_max"] <= LSE_ABS, f"{what}: {stats}"
    return stats


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def small(name="t", *, B=1, H=2, Hkv=None, S=200, Sq=None, Skv=None, D=64, dtype="bf16",
          causal=False, window=0, documents=False, mod="none", softcap=30.0, seed=7,
          doc_range=(16, 96), q_offset=0, prefix=None, rel_max=0) -> Inputs:
    """Small seeded inputs (Sq and Skv may differ; query row i at key
    position i + q_offset)."""
    from workload import (alibi_slopes, as_element_type, document_ids, document_lengths, draw_qkv,
                          rel_bias_table)
    Hkv = Hkv or H
    Sq = Sq or S
    Skv = Skv or S
    wl = Workload(name, B=B, H=H, Hkv=Hkv, S=S, D=D, dtype=dtype, causal=causal, window=window,
                  documents=documents, mod=mod, softcap=softcap, seed=seed, doc_seed=seed,
                  doc_len_range=doc_range, q_offset=q_offset, prefix=prefix, rel_max=rel_max)
    q, k, v = draw_qkv(B, H, Hkv, Sq, Skv, D, seed)
    q, k, v = (as_element_type(t, dtype) for t in (q, k, v))
    doc = None
    if documents:
        n = max(Sq + q_offset, Skv)
        doc = np.stack([document_ids(document_lengths(n, seed + b, *doc_range)) for b in range(B)])
    slopes = alibi_slopes(H) if mod == "alibi" else None
    rel = rel_bias_table(H, rel_max, seed) if mod == "relbias" else None
    return Inputs(_SqSkv(wl, Sq, Skv), q, k, v, doc, slopes, rel_bias=rel)


class _SqSkv:
    """A Workload view with Sq != Skv."""

    def __init__(self, wl: Workload, Sq: int, Skv: int):
        self._wl, self.Sq, self.Skv = wl, Sq, Skv

    def __getattr__(self, name):
        return getattr(self._wl, name)


__all__ = ["run_gpu", "run_oracle", "run_oracle_full", "compare", "to_np", "small", "make_inputs",
           "device_variant", "oracle_kwargs"]
