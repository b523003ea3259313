"""Scalar pure-Python attention: a second, independent reading of the
definition, used only to check the vectorised oracle on tiny shapes.

Every score is a Python float computed with explicit loops and math.exp /
math.tanh; nothing here is shared with the oracle.
"""
import math


def brute_attention(q, k, v, scale, *, causal=False, window=None, doc_ids=None,
                    alibi_slopes=None, softcap=None, q_offset=0, prefix=None, rel_bias=None):
    """q: nested lists [B][H][Sq][D]; k, v: [B][Hkv][Skv][D]. Returns nested
    lists O [B][H][Sq][D] and LSE [B][H][Sq]. Query i stands at key position
    i + q_offset; with `prefix` the keys before it are exempt from causality."""
    B, H, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Skv = len(k[0]), len(k[0][0])
    O = [[[[0.0] * D for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h * Hkv // H          # query heads split into Hkv equal consecutive groups
            for i in range(Sq):
                p = i + q_offset
                kept = []
                for j in range(Skv):
                    in_prefix = prefix is not None and j < prefix
                    if causal and j > p and not in_prefix:
                        continue
                    if window and p - j >= window:
                        continue
                    if doc_ids is not None and doc_ids[b][p] != doc_ids[b][j]:
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += q[b][h][i][d] * k[b][g][j][d]
                    s = dot * scale
                    if alibi_slopes is not None:
                        s = s + alibi_slopes[h] * (j - p)
                    if rel_bias is not None:
                        R = (len(rel_bias[h]) - 1) // 2
                        d = j - p
                        d = -R if d < -R else (R if d > R else d)
                        s = s + rel_bias[h][d + R]
                    if softcap is not None:
                        s = softcap * math.tanh(s / softcap)
                    kept.append((j, s))
                if not kept:
                    L[b][h][i] = -math.inf
                    continue
                top = max(s for _, s in kept)
                ws = [(j, math.exp(s - top)) for j, s in kept]
                tot = sum(w for _, w in ws)
                for d in range(D):
                    O[b][h][i][d] = sum(w * v[b][g][j][d] for j, w in ws) / tot
                L[b][h][i] = top + math.log(tot)
    return O, L
