"""Oracle: plain, slow, fp64 CPU attention forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it and
shares no code with it.

What it computes. The fused, tiled method reorganises where the work happens
but approximates nothing, so its result is the plain one and accuracy is not
traded for speed (Neuron FA4 explainer, "Enter Tri Dao and FlashAttention",
and its TL;DR). So the oracle is the unfused definition of attention written
out, comparing every query with every key (same page, "What Is Attention, and
Why Is It Expensive?"), with the score modification and the mask that
FlexAttention lets a user attach to a (query index, key index) pair applied
literally (NextVector FlexAttention article, body: a function of q_idx and
k_idx modifies the score; PyTorch FlexAttention FA4-backend post: user
functions that modify scores or mask pairs out):

    s[q, j]  = scale * <Q[b, h, q, :], K[b, kvh(h), j, :]>
    s'[q, j] = score_mod(s[q, j], b, h, q, j)
    admitted = { j : mask_mod(b, h, q, j) }
    O[q]     = sum_{j admitted} exp(s'[q, j]) V[b, kvh(h), j, :] / sum_{j admitted} exp(s'[q, j])
    LSE[q]   = log sum_{j admitted} exp(s'[q, j])

with a row whose admitted set is empty defined as O = 0, LSE = -inf.

The whole score row is materialised in fp64 (the very N x N matrix the fused
method keeps out of HBM: NextVector article, "Executive Key Takeaways"), the
softmax is taken with the row maximum subtracted once (an exact identity, used
only to keep exp() finite), and nothing is blocked, fused or reordered.

Readings where the pages are silent (each also listed in the design notes):
  * the scale multiplies the raw dot product before the score modification;
  * mask and modification see (b, h, q_idx, k_idx); a masked score is -inf after
    the modification, so the mask always wins;
  * causal is q_idx >= k_idx, the sliding window is q_idx - k_idx < window, and
    documents admit a pair iff both positions carry the same document label;
    several masks compose by AND;
  * ALiBi adds slope[h] * (k_idx - q_idx) to the scaled score; soft-capping
    replaces it by c * tanh(s / c);
  * relative position bias (the PyTorch 2.5 / FlexAttention article names
    relative position encodings among its variants without a form): a
    per-head table of 2R + 1 values added to the scaled score, indexed by
    k_idx - q_idx clipped to [-R, R]; ALiBi is the linear table with R at
    least the sequence length;
  * grouped heads: query head h reads key/value head h // (H // Hkv).
  * query row i stands at key position i + q_offset (0 by default, so rows and
    keys start together); masks, ALiBi distances and document labels see that
    position. Decoding and chunked prefill after Skv - Sq cached keys take
    q_offset = Skv - Sq (the pages name Sq != Skv work only as a direction);
  * prefix masking (named, not defined, in the PyTorch 2.5 / FlexAttention
    article's overview and "What Happened?"): with causal, the keys before
    `prefix` are visible to every query, the causal rule holds for the rest,
    and the other masks still compose by AND.

Every function here is pinned by tests that do not reuse it (closed forms,
invariants, a scalar brute force and a library routine).
"""
from __future__ import annotations

import numpy as np

__all__ = ["kv_head_of", "admitted", "modified_scores", "attention", "attention_backward",
           "pair_count", "tile_classes"]


def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """Grouped heads: H // Hkv consecutive query heads share one K/V head."""
    if H % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return h // (H // Hkv)


def admitted(q_idx, k_idx, *, causal: bool = False, window: int | None = None,
             doc_row=None, prefix: int | None = None) -> np.ndarray:
    """The mask: True where the query at position q_idx may attend to the key
    at position k_idx.

    `q_idx`, `k_idx` broadcast against each other (e.g. a column and a row of
    positions); `doc_row` is the document label of every position of one
    batch row (or None). `prefix` (prefix-LM, with causal): keys before it
    are visible to every query, the causal rule applies from it on.
    """
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    keep = np.ones(np.broadcast_shapes(q_idx.shape, k_idx.shape), dtype=bool)
    if causal:
        c = q_idx >= k_idx
        if prefix is not None and prefix > 0:
            c = c | (k_idx < prefix)
        keep &= c
    if window is not None and window > 0:
        keep &= (q_idx - k_idx) < window
    if doc_row is not None:
        doc_row = np.asarray(doc_row)
        keep &= doc_row[q_idx] == doc_row[k_idx]
    return keep


def modified_scores(s: np.ndarray, h: int, q_idx, k_idx, *, alibi_slopes=None,
                    softcap: float | None = None, rel_bias=None) -> np.ndarray:
    """The score modification applied to already-scaled scores `s`.

    rel_bias: [H, 2R + 1] table; the bias of a pair is the entry of its
    relative position k_idx - q_idx clipped to [-R, R] (entry index
    clip + R)."""
    if sum(x is not None for x in (alibi_slopes, softcap, rel_bias)) > 1:
        raise ValueError("one score modification at a time")
    if rel_bias is not None:
        tab = np.asarray(rel_bias, dtype=np.float64)[h]
        R = (tab.shape[0] - 1) // 2
        dist = np.asarray(k_idx, dtype=np.int64) - np.asarray(q_idx, dtype=np.int64)
        return s + tab[np.clip(dist, -R, R) + R]
    if alibi_slopes is not None:
        slope = float(np.asarray(alibi_slopes, dtype=np.float64)[h])
        dist = np.asarray(k_idx, dtype=np.float64) - np.asarray(q_idx, dtype=np.float64)
        return s + slope * dist
    if softcap is not None:
        c = float(softcap)
        return c * np.tanh(s / c)
    return s


def attention(q, k, v, scale: float, *, causal: bool = False, window: int | None = None,
              doc_ids=None, alibi_slopes=None, softcap: float | None = None, rows=None,
              heads=None, q_offset: int = 0, prefix: int | None = None, rel_bias=None):
    """fp64 attention forward, the definition written out.

    q: [B, H, Sq, D], k and v: [B, Hkv, Skv, D] (any real dtype; computed in
    float64). Query row i sits at position i + q_offset of the key sequence
    (masks, score mods and document labels see positions). doc_ids:
    [B, >= max(Sq + q_offset, Skv)] document label per position, or None.
    prefix: prefix-LM boundary (see `admitted`). rows: optional 1-D array of
    query indices to evaluate (for sampled checks at full size); heads:
    optional list of query heads to evaluate.

    Returns (O, LSE): O [B, H, len(rows), D] float64 and LSE [B, H, len(rows)]
    float64 (natural log). Heads not in `heads` are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(H) if heads is None else heads
    keys = np.arange(Skv)

    O = np.full((B, H, rows.size, D), np.nan)
    LSE = np.full((B, H, rows.size), np.nan)
    for b in range(B):
        doc_row = None if doc_ids is None else np.asarray(doc_ids)[b]
        pos = rows + q_offset
        keep = admitted(pos[:, None], keys[None, :], causal=causal, window=window,
                        doc_row=doc_row, prefix=prefix)
        any_kept = keep.any(axis=1)
        for h in heads:
            kh = kv_head_of(h, H, Hkv)
            s = (q[b, h, rows, :] @ k[b, kh].T) * scale
            s = modified_scores(s, h, pos[:, None], keys[None, :],
                                alibi_slopes=alibi_slopes, softcap=softcap, rel_bias=rel_bias)
            s = np.where(keep, s, -np.inf)
            m = np.where(any_kept, s.max(axis=1, initial=-np.inf), 0.0)
            w = np.exp(s - m[:, None])          # exp(-inf) = 0 for masked keys
            l = w.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                o = (w @ v[b, kh]) / l[:, None]
                lse = m + np.log(l)
            O[b, h] = np.where(any_kept[:, None], o, 0.0)
            LSE[b, h] = np.where(any_kept, lse, -np.inf)
    return O, LSE


def attention_backward(q, k, v, dout, scale: float, *, causal: bool = False,
                       window: int | None = None, doc_ids=None, alibi_slopes=None,
                       softcap: float | None = None, q_offset: int = 0,
                       prefix: int | None = None, rel_bias=None):
    """fp64 gradients of the attention forward: for the loss L = sum(O * dout),
    returns (dQ, dK, dV) with the shapes of q, k and v.

    The pages name a backward pass (used in training, reproducible in FA4's
    deterministic mode: Neuron FA4 explainer, "FlashAttention-4: Built for
    Blackwell", backward-pass fixes) but give no formulas; this is the exact
    derivative of the definition in `attention`, written out row by row:

        P      = softmax of the admitted modified scores (0 where masked,
                 and a row with no admitted key has P = 0 and O = 0)
        dV    += P^T dout                      (summed over the query heads of a group)
        dP     = dout V^T
        dS'    = P * (dP - rowsum(P * dP))     (the softmax Jacobian applied to dP)
        dS     = dS' * d s' / d s              (1 for no mod, ALiBi and relative bias; 1 - tanh^2(s / c) for soft-capping)
        dQ     = scale * dS K,   dK += scale * dS^T Q
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    if dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("shape mismatch")
    rows, keys = np.arange(Sq), np.arange(Skv)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        doc_row = None if doc_ids is None else np.asarray(doc_ids)[b]
        pos = rows + q_offset
        keep = admitted(pos[:, None], keys[None, :], causal=causal, window=window, doc_row=doc_row,
                        prefix=prefix)
        any_kept = keep.any(axis=1)
        for h in range(H):
            kh = kv_head_of(h, H, Hkv)
            s = (q[b, h] @ k[b, kh].T) * scale
            sm = modified_scores(s, h, pos[:, None], keys[None, :], alibi_slopes=alibi_slopes,
                                 softcap=softcap, rel_bias=rel_bias)
            sm = np.where(keep, sm, -np.inf)
            m = np.where(any_kept, sm.max(axis=1, initial=-np.inf), 0.0)
            w = np.exp(sm - m[:, None])
            l = w.sum(axis=1)
            P = np.where(any_kept[:, None], w / np.where(l > 0, l, 1.0)[:, None], 0.0)
            dV[b, kh] += P.T @ dout[b, h]
            dP = dout[b, h] @ v[b, kh].T
            dSm = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            if softcap is not None:
                dS = dSm * (1.0 - np.tanh(s / float(softcap)) ** 2)
            else:
                dS = dSm
            dQ[b, h] = scale * (dS @ k[b, kh])
            dK[b, kh] += scale * (dS.T @ q[b, h])
    return dQ, dK, dV


def pair_count(Sq: int, Skv: int, *, causal: bool = False, window: int | None = None,
               doc_row=None, q_offset: int = 0, prefix: int | None = None) -> int:
    """Number of admitted (query, key) pairs, counted element by element."""
    total = 0
    keys = np.arange(Skv)
    for lo in range(0, Sq, 1024):
        r = np.arange(lo, min(Sq, lo + 1024)) + q_offset
        total += int(admitted(r[:, None], keys[None, :], causal=causal,
                              window=window, doc_row=doc_row, prefix=prefix).sum())
    return total


def tile_classes(Sq: int, Skv: int, tile: int, *, causal: bool = False,
                 window: int | None = None, doc_row=None, q_offset: int = 0,
                 prefix: int | None = None) -> np.ndarray:
    """Classify every (query tile, key tile) pair by testing every pair of
    positions: 0 = empty (no admitted pair), 2 = full (every query row in
    range admits every key of the tile, and the tile lies inside [0, Skv)),
    1 = partial otherwise. Query rows past Sq are ignored; keys past Skv never
    exist, so a tile reaching past Skv is never full.

    Returns int array [ceil(Sq/tile), ceil(Skv/tile)].
    """
    nq, nk = -(-Sq // tile), -(-Skv // tile)
    out = np.zeros((nq, nk), dtype=np.int64)
    for i in range(nq):
        rows = np.arange(i * tile, min(Sq, (i + 1) * tile))
        keep = admitted(rows[:, None] + q_offset, np.arange(Skv)[None, :], causal=causal,
                        window=window, doc_row=doc_row, prefix=prefix)
        for j in range(nk):
            blk = keep[:, j * tile:(j + 1) * tile]
            if not blk.any():
                out[i, j] = 0
            elif blk.all() and (j + 1) * tile <= Skv:
                out[i, j] = 2
            else:
                out[i, j] = 1
    return out
