"""Pure-Python brute-force attention for tiny inputs.

TEST INFRASTRUCTURE. It pins ``oracle.attention`` on small cases: it shares
none of that module's code and uses no array library, only per-query loops
over an explicit list of allowed keys and ``math.exp``.

Allowed keys follow the same reading of the RFC's Generalized Causal
Attention ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0 and Model
structure item 1): for a text query at position i the keys are positions
0..i; for an image query they are every position of its sequence.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def allowed_keys(i: int, text_len: int, seq_len: int) -> List[int]:
    if i < text_len:
        return list(range(i + 1))
    return list(range(seq_len))


def attend_one(qrow: Sequence[float], keys: Sequence[Sequence[float]], vals: Sequence[Sequence[float]],
               allowed: Sequence[int], scale: float) -> List[float]:
    """Softmax-weighted average of vals over ``allowed`` for a single query row."""
    D = len(qrow)
    if not allowed:
        return [0.0] * len(vals[0]) if vals else []
    logits = []
    for j in allowed:
        dot = 0.0
        for d in range(D):
            dot += float(qrow[d]) * float(keys[j][d])
        logits.append(scale * dot)
    top = max(logits)
    weights = [math.exp(x - top) for x in logits]
    total = math.fsum(weights)
    Dv = len(vals[0])
    out = []
    for d in range(Dv):
        acc = math.fsum(w * float(vals[j][d]) for w, j in zip(weights, allowed))
        out.append(acc / total)
    return out


def brute_packed_attention(q, k, v, text_len: Sequence[int], image_len: Sequence[int],
                           scale: float) -> List[List[List[float]]]:
    """q, k, v indexable as [N][H][D]; returns nested lists [N][H][D]."""
    N = len(q)
    H = len(q[0]) if N else 0
    out = [[None] * H for _ in range(N)]
    start = 0
    for T, I in zip(text_len, image_len):
        L = int(T) + int(I)
        for h in range(H):
            keys = [k[start + j][h] for j in range(L)]
            vals = [v[start + j][h] for j in range(L)]
            for i in range(L):
                out[start + i][h] = attend_one(q[start + i][h], keys, vals,
                                               allowed_keys(i, int(T), L), scale)
        start += L
    if start != N:
        raise ValueError("token count does not match the sequence lengths")
    return out
