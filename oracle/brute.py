"""Pure-Python brute-force attention for tiny inputs.

TEST INFRASTRUCTURE. It pins ``oracle.attention`` on small cases: it shares
none of that module's code and uses no array library, only per-query loops
over an explicit list of allowed keys and ``math.exp``.

Allowed keys follow the same reading of the RFC's Generalized Causal
Attention ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0 and Model
structure item 1): for a text query at position i the keys are positions
0..i; for an image query they are every position of its sequence. For
sequences of several text and image segments (pinning ``oracle.segments``)
the allowed keys are characterised differently from that module, as "not
later than the query, or inside the query's own image block".
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


def segment_allowed_keys(i: int, seg_len: Sequence[int], seg_kind: Sequence[int]) -> List[int]:
    """Keys a query at position i may see, by a second characterisation of
    the multi-segment Generalized Causal mask: key j is allowed when it is not
    later than i, or when i lies in an image (FULL, kind 1) block and j lies in
    that same block."""
    bounds = []
    a = 0
    for n in seg_len:
        bounds.append((a, a + int(n)))
        a += int(n)
    L = a
    seg_of = [None] * L
    for sidx, (lo, hi) in enumerate(bounds):
        for p in range(lo, hi):
            seg_of[p] = sidx
    out = []
    for j in range(L):
        same_full_block = seg_kind[seg_of[i]] == 1 and seg_of[j] == seg_of[i]
        if j <= i or same_full_block:
            out.append(j)
    return out


def brute_segment_attention(q, k, v, seqs, scale: float) -> List[List[List[float]]]:
    """q indexable as [Nq][H][D] (queried rows only: positions q_start..L-1 of
    each sequence, packed in order), k, v as [Nk][H][D]; each entry of
    ``seqs`` has seg_len, seg_kind and q_start. Returns nested lists [Nq][H][D]."""
    Nq = len(q)
    H = len(q[0]) if Nq else 0
    out = [[None] * H for _ in range(Nq)]
    kstart = qstart = 0
    for s in seqs:
        L = sum(int(n) for n in s.seg_len)
        for h in range(H):
            keys = [k[kstart + j][h] for j in range(L)]
            vals = [v[kstart + j][h] for j in range(L)]
            for i in range(int(s.q_start), L):
                r = qstart + i - int(s.q_start)
                out[r][h] = attend_one(q[r][h], keys, vals, segment_allowed_keys(i, s.seg_len, s.seg_kind), scale)
        kstart += L
        qstart += L - int(s.q_start)
    if qstart != Nq:
        raise ValueError("query count does not match the sequences")
    return out
